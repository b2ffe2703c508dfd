// A4a / A4b - dispatch permute into a rank-contiguous send buffer.
//
// Source: "Expert Coupling in MoE Pretraining" (summary), "Method 1: Correlated
// Expert Placement + Deduplicating Dispatcher".  Plain dispatch repeats a
// token's row for every expert it selected; the deduplicating variant writes
// the row once per rank the token needs and attaches to it the ids and gates
// of all the token's experts on that rank.  "DODOCO" dataset card, "Reading
// the counts": the plain counts (and rows) repeat a token for each of its
// experts, also when several of them share a rank.
//
// Design: one wave per (token, row chunk).  The wave reads its chunk of x[t]
// once into registers (16-byte loads, 1 KiB per wave instruction) while lanes
// j < k resolve slot j's destination row from the plan (the tile's first row in
// the slot's column + the slot's rank inside the tile), then writes the chunk
// to each destination row.  Every access is a full, contiguous row segment, so
// reads and writes are perfectly coalesced.  Each wave then writes the row
// metadata of one token, in a token order that keeps a token range's metadata
// on one XCD (meta_block below).
#include "common.hpp"
#include "coselect_bm.hpp"
#include "plan_order.hpp"

namespace moe {

// Loads are issued unconditionally from addresses clamped into the row, so a
// wave's loads go out back to back (a load under a lane-divergent branch is
// followed by a wait for it); only the stores are predicated.  They are
// nontemporal: a call reads each row once, and keeping those reads out of the
// caches leaves the Infinity Cache to the rows just written, which the combine
// (or, on the receive side, the reduction) reads next.  Whole steps 1-6%
// faster (16384-token top-2 receive step 287 -> 270 us, 4096-token top-8 step
// at 256 experts 53.1 -> 51.8 us), though a 4096-token top-6 dispatch timed
// alone, back to back, is 1.6% slower.
template <int NV>
__device__ __forceinline__ void load_chunk(u32x4 (&v)[NV], const uint8_t* row, int64_t chunk0,
                                           int row_bytes, int lane) {
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int64_t off = chunk0 + int64_t(i * kWave + lane) * 16;
    off = off < row_bytes ? off : row_bytes - 16;
    v[i] = load16_nt(row + off);
  }
}

// Keeps the row loads above it ahead of what follows.  Without it the compiler
// issues them after the position lookups (slot code, then the tile's counts),
// so each wave waits for three memory round trips in a row instead of
// overlapping the row with the lookups.  The row pointer `x` of the kernels is
// deliberately not __restrict__ (nor the plan tables `lslot`, `gbase`,
// `tcnt`): loads through a restrict read-only pointer count as invariant, and
// the compiler moves those past the fence.
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

// Makes `v` available here.  The metadata values are computed before the row
// stores: computed after them (where the compiler would sink them), the wait
// for their loads would also wait for every row store issued since.
__device__ __forceinline__ void ready(int v) { asm volatile("" ::"v"(v)); }

// First row of position column `col` in tile b: the scan's base of the tile's
// 16-tile group plus the counts of the group's earlier tiles (one 16-byte load
// of the column's tile counts).
__device__ __forceinline__ int tile_first_row(const int32_t* gbase,
                                              const uint8_t* tcnt, int64_t Bp,
                                              int64_t G, int tcol, int col, int64_t b) {
  const int g = int(gbase[col * G + (b >> 4)]);
  const u32x4 tv = load16(tcnt + tcol * Bp + (b & ~int64_t(15)));
  return g + byte_sum(keep_bytes(tv, int(b & 15)));
}

// ------------------------------------------ plans scanned by the dispatch --
//
// For a plan of at most kEmbedMaxVec 16-tile vectors of position-column tile
// counts (the expert columns; the rank columns in dedup mode) the dispatch
// workgroups do the plan's scan themselves, so the routing call needs no scan
// launch of its own (moe_route_dispatch): every workgroup reads the position
// columns' tile counts (L2 hits: 8 KiB at 4096 tokens and 64 experts, 16 KiB
// for 32 ranks at 16384 tokens), takes every such column's total and group
// prefixes in LDS, orders and scans the columns (order_columns, as the scan
// kernel does), and looks its rows' positions up in LDS.  The tile-count loads
// are issued before the row loads (a wave's loads complete in order), so the
// scan runs while the rows are in flight; all of them, four per thread (eight
// for plans of more than 1024 vectors), go out at once, since any load issued
// after the rows would make the scan wait for the rows.  Workgroup 0 also
// writes the counts, offsets, header and group bases, so the workspace then
// holds the same plan as after the scan kernel; in dedup mode it also adds up
// the expert columns for the per-expert counts, which no other workgroup needs
// (loads issued after its rows: only workgroup 0 waits for them).
constexpr int kEmbedMaxVec = 2048;
// ... and at most this many tile-count vectors summed over the dispatch's copy
// workgroups (each reads them all, 16 bytes each: 64 MiB of L2 reads).  The
// scan costs the dispatch more the more of them there are: at 16384 tokens of
// 8 KiB rows (8192 workgroups), +2.5 us for 8 ranks (256 vectors: 32 MiB, a
// net 2.7 us gain on the 110 us top-2 dedup step) but +5.6 us for 32 ranks
// (1024 vectors: 128 MiB), as much as the scan kernel it replaces (5.4 us), and
// that top-6 step ran 11 us slower with two batches overlapped on two streams.
constexpr int64_t kEmbedMaxVecBlocks = int64_t(4) << 20;

// The dispatch kernels' scan variant: 0 none (bases from the workspace); 1 / 2
// four vectors per thread, contiguous / explicit placement; 3 / 4 eight.
constexpr bool sc_ranked(int sc) { return sc == 2 || sc == 4; }
constexpr int sc_vectors(int sc) { return sc >= 3 ? 8 : 4; }

struct ScanArgs {
  int B;                    // tiles
  int E, R, m;              // experts, ranks, experts per rank (contiguous placement)
  const int32_t* place;     // expert -> rank (explicit placement, plain dispatch)
  int32_t* expert_counts;
  int32_t* rank_counts;
  int32_t* rank_offsets;
  int32_t* expert_offsets;  // may be null
  int32_t* header;
  int32_t* gbase;           // the plan's group bases, written by workgroup 0
};

// Dynamic LDS of scan_small_plan: s_tot[C], s_col[E], s_pre[CP * G], OrderLds
// (C columns counted, CP of them position columns).
__host__ __device__ inline size_t scan_head_bytes(int C, int CP, int E, int G) {
  const size_t head = (size_t(C) + size_t(E) + size_t(CP) * size_t(G)) * 4;
  return (head + 7) / 8 * 8;
}
template <bool RANKED>
__host__ __device__ inline size_t scan_lds_bytes(int C, int CP, int E, int G) {
  return scan_head_bytes(C, CP, E, G) + sizeof(OrderLds<RANKED>);
}

// The loads of scan_small_plan, issued by the dispatch kernels before their
// row loads: N 16-tile vectors of the position columns per thread.
template <int N>
struct ScanPrefetch {
  u32x4 vv[N];
  int my_rank;  // RANKED: the rank of expert threadIdx.x
};

// cbase, CP: the tcnt column of position column 0 and the position columns.
template <bool RANKED, int N>
__device__ __forceinline__ void scan_prefetch(const uint8_t* tcnt, int G, int cbase, int CP,
                                              const ScanArgs& a, ScanPrefetch<N>& pf) {
  const int tid = threadIdx.x;
  const int V = CP * G;
  const u32x4* g4 = reinterpret_cast<const u32x4*>(tcnt) + int64_t(cbase) * G;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int q = tid + i * int(blockDim.x);
    pf.vv[i] = g4[q < V ? q : V - 1];
  }
  pf.my_rank = (RANKED && tid < a.E) ? clampi(a.place[tid], 0, a.R - 1) : 0;
}

// Every thread of the workgroup calls it (blockDim.x >= max(CP, R), and E
// when RANKED or, in dedup mode, with `outputs`), after scan_prefetch.  Leaves
// s_col[p] = the first row of position column p (the expert id when RANKED)
// and s_pre[p * G + g] = the rows of position column p in the groups before g;
// returns the total number of rows.
template <bool DEDUP, bool RANKED, int N>
__device__ __forceinline__ int scan_small_plan(const uint8_t* tcnt, int G, const ScanArgs& a,
                                               const ScanPrefetch<N>& pf, bool outputs,
                                               uint8_t* lds, int32_t*& s_col, int32_t*& s_pre) {
  const int E = a.E, R = a.R;
  const int C = E + (DEDUP ? R : 0);
  const int cbase = DEDUP ? E : 0;
  const int CP = DEDUP ? R : E;
  int32_t* s_tot = reinterpret_cast<int32_t*>(lds);
  s_col = s_tot + C;
  s_pre = s_col + E;
  OrderLds<RANKED>& L =
      *reinterpret_cast<OrderLds<RANKED>*>(lds + scan_head_bytes(C, CP, E, G));
  const int tid = threadIdx.x;
  const int V = CP * G;
  // byte sums of every 16-tile vector (V <= N * blockDim.x: all prefetched)
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int q = tid + i * int(blockDim.x);
    if (q < V) s_pre[q] = byte_sum(keep_bytes(pf.vv[i], a.B - 16 * (q % G)));
  }
  order_init<RANKED>(L);
  const bool expert_sums = DEDUP && outputs;  // the per-expert counts (workgroup 0)
  if (expert_sums && tid < E) s_tot[tid] = 0;
  __syncthreads();
  // each position column's total and exclusive prefix over its groups
  for (int p = tid; p < CP; p += blockDim.x) {
    int run = 0;
    for (int g = 0; g < G; ++g) {
      const int x = s_pre[p * G + g];
      s_pre[p * G + g] = run;
      run += x;
    }
    s_tot[cbase + p] = run;
  }
  if (expert_sums) {  // four loads in flight per thread, then their sums
    const u32x4* g4 = reinterpret_cast<const u32x4*>(tcnt);
    const int EV = E * G, nt = blockDim.x;
    for (int q0 = tid; q0 < EV; q0 += 4 * nt) {
      u32x4 ev[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ev[i] = g4[q0 + i * nt < EV ? q0 + i * nt : EV - 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = q0 + i * nt;
        if (q < EV) atomicAdd(&s_tot[q / G], byte_sum(keep_bytes(ev[i], a.B - 16 * (q % G))));
      }
    }
  }
  __syncthreads();
  const int total = order_columns<DEDUP, RANKED>(s_tot, s_col, L, E, R, a.m, pf.my_rank, outputs,
                                                 a.expert_counts, a.rank_counts, a.rank_offsets,
                                                 a.expert_offsets, a.header);
  if (outputs)
    for (int i = tid; i < V; i += blockDim.x) a.gbase[i] = s_col[i / G] + s_pre[i];
  return total;
}

// First row of position column `col` (tcnt column `tcol`) in tile b, from the
// LDS tables of scan_small_plan.
__device__ __forceinline__ int lds_first_row(const int32_t* s_col, const int32_t* s_pre,
                                             const uint8_t* tcnt, int64_t Bp, int64_t G,
                                             int tcol, int col, int64_t b) {
  const u32x4 tv = load16(tcnt + tcol * Bp + (b & ~int64_t(15)));
  return s_col[col] + s_pre[col * G + (b >> 4)] + byte_sum(keep_bytes(tv, int(b & 15)));
}

template <int NV, bool NT>
__device__ __forceinline__ void store_chunk(const u32x4 (&v)[NV], uint8_t* dst, int64_t chunk0,
                                            int row_bytes, int lane) {
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int64_t off = int64_t(i * kWave + lane) * 16;
    if (chunk0 + off < row_bytes) {
      if (NT)
        store16_nt(dst + off, v[i]);
      else
        store16(dst + off, v[i]);
    }
  }
}

// Logical block whose token metadata this block's waves write (META): the
// hardware hands consecutive workgroups to the 8 XCDs in
// turn, so the rows of a token range are copied by every XCD at once (the
// order that suits the row writes), while the metadata of the range - 4-byte
// entries that neighbouring tokens share cache lines in - is written from one
// XCD, whose L2 then merges the partial lines: XCD x writes the metadata of
// the logical blocks [x*n/8, (x+1)*n/8).  The grid is a multiple of 8 blocks,
// so this is a bijection and every token's metadata is written once.
// Without META (small grids, where every wave waits on latency rather than
// bandwidth, and the receive-side expansion, measured slower with it) each
// wave writes the metadata of its own token.
// bid, nb: this block and the number of copy blocks (the grid without the
// co-selection blocks in front, a multiple of 8 of them).
template <bool META>
__device__ __forceinline__ int64_t meta_block(unsigned bid, unsigned nb) {
  if (!META) return bid;
  const unsigned per = nb >> 3;
  return int64_t(bid & 7u) * per + (bid >> 3);
}

// With cs_blocks > 0 the first cs_blocks workgroups (a multiple of 8, so the
// copy blocks keep their XCD order) take the co-selection counts of the plan's
// expert bitmaps instead: their loads and popcounts overlap the row copies,
// which are bound by HBM.  Returns true in those workgroups.
__device__ __forceinline__ bool coselect_part(const CoselectBm& cs, int cs_blocks) {
  if (int(blockIdx.x) >= cs_blocks) return false;
  extern __shared__ uint64_t s_cs[];
  if (int64_t(blockIdx.x) < cs.blocks()) coselect_bm_block(cs, blockIdx.x, s_cs);
  return true;
}

// PAD: the receive-side expansion, where a "token" is a received row, slots
// with the code kNoSlot are empty, only rows below *n_valid are expanded, and
// no row is written at or past out_cap (such slots get slot_row = -1).
//
// Each wave copies the row chunk of (token t, chunk c) and writes the metadata
// of token tm (when its wave index in the metadata order is chunk 0 of tm).
// Every load of both is issued before the first wait, from in-bounds indices.
// SC: 0 = group bases from the workspace; else the workgroups scan the plan
// (sc_ranked, sc_vectors).
template <int NV, bool NT, bool PAD, bool META, int SC>
__global__ void __launch_bounds__(256)
dispatch_kernel(const uint8_t* x, const float* __restrict__ gate, int64_t T,
                int row_bytes, int k, int cpr, const int32_t* gbase,
                const uint8_t* tcnt, const uint32_t* lslot, int64_t Bp,
                int64_t G, uint8_t* __restrict__ send,
                int32_t* __restrict__ row_token, int32_t* __restrict__ row_expert,
                float* __restrict__ row_weight, int32_t* __restrict__ slot_row,
                const int32_t* __restrict__ n_valid, int64_t out_cap, CoselectBm cs,
                int cs_blocks, ScanArgs sa) {
  static_assert(!(PAD && SC), "the expansion's plan comes from its scan kernel");
  if (coselect_part(cs, cs_blocks)) return;
  const unsigned bid = blockIdx.x - unsigned(cs_blocks), nb = gridDim.x - unsigned(cs_blocks);
  const int lane = lane_id();
  // lanes j < k own slot j; the other lanes load slot k-1's data and ignore it
  const int jl = lane < k ? lane : k - 1;
  const int64_t nv = PAD ? int64_t(*n_valid) : T;
  const int64_t wid = (int64_t(bid) * blockDim.x + threadIdx.x) / kWave;
  const int64_t t = wid / cpr;
  const int64_t wm = (meta_block<META>(bid, nb) * blockDim.x + threadIdx.x) / kWave;
  const int64_t tm = wm / cpr;
  static_assert(!(PAD && META), "the expansion writes the metadata of its own rows");
  const int c = int(wid - t * cpr);
  if (PAD && t < T && t >= nv) {  // whole wave: a row past the received ones
    if (c == 0 && lane < k) slot_row[t * k + lane] = -1;
    return;
  }
  const bool copy = t < T && t < nv;            // wave-uniform
  const bool meta = tm < T && wm == tm * cpr;   // wave-uniform: one wave per token
  if (!SC && !copy && !meta) return;            // (with SC every wave takes the scan's barriers)
  // The loads are unconditional, from tokens in range: a load under a branch
  // the compiler cannot prove uniform is followed by a wait for it.
  const int64_t tl = copy ? t : (meta ? tm : T - 1);
  const int64_t tml = meta ? tm : tl;
  const int64_t chunk0 = int64_t(c) * (NV * kWave * 16);
  const uint32_t code = lslot[tl * k + jl];  // (expert << 8) | rank inside the tile
  const uint32_t code_m = META ? lslot[tml * k + jl] : code;
  const float g_m = gate[tml * k + jl];
  ScanPrefetch<sc_vectors(SC)> pf;
  if (SC) {
    scan_prefetch<sc_ranked(SC)>(tcnt, int(G), 0, sa.E, sa, pf);
    issue_fence();
  }
  u32x4 v[NV];
  load_chunk<NV>(v, x + tl * row_bytes, chunk0, row_bytes, lane);
  issue_fence();
  int32_t* s_col = nullptr;
  int32_t* s_pre = nullptr;
  if (SC) {
    extern __shared__ uint64_t s_scan[];
    scan_small_plan<false, sc_ranked(SC)>(tcnt, int(G), sa, pf, bid == 0,
                                          reinterpret_cast<uint8_t*>(s_scan), s_col, s_pre);
    if (!copy && !meta) return;
  }
  const bool has = !PAD || code != kNoSlot;
  const int e = has ? int(code >> 8) : 0;
  const int pos = (SC ? lds_first_row(s_col, s_pre, tcnt, Bp, G, e, e, tl / kTile)
                      : tile_first_row(gbase, tcnt, Bp, G, e, e, tl / kTile)) +
                  int(code & 255u);
  const bool has_m = !PAD || code_m != kNoSlot;
  const int e_m = has_m ? int(code_m >> 8) : 0;
  const int pos_m =
      META ? (SC ? lds_first_row(s_col, s_pre, tcnt, Bp, G, e_m, e_m, tml / kTile)
                 : tile_first_row(gbase, tcnt, Bp, G, e_m, e_m, tml / kTile)) +
                 int(code_m & 255u)
           : pos;
  issue_fence();
  ready(pos_m);
  if (copy) {
    const bool ok = has && (!PAD || pos < out_cap);
    const uint64_t okm = __ballot(lane < k && ok);
    for (int j = 0; j < k; ++j) {
      if (PAD && !((okm >> j) & 1ull)) continue;
      const int p = bcast(pos, j);
      store_chunk<NV, NT>(v, send + int64_t(p) * row_bytes + chunk0, chunk0, row_bytes, lane);
    }
  }
  // metadata after the row stores: stores count against the same wait counter
  // as loads, so stores issued first would hold up the rows
  if (meta && lane < k) {
    const bool ok = has_m && (!PAD || pos_m < out_cap);
    slot_row[tm * k + lane] = ok ? pos_m : -1;
    if (ok) {
      row_token[pos_m] = int32_t(tm);
      row_expert[pos_m] = e_m;
      row_weight[pos_m] = g_m;
    }
  }
}

// SC: the workgroups scan the plan (see dispatch_kernel; never ranked).
template <int NV, bool NT, bool META, int SC>
__global__ void __launch_bounds__(256)
dispatch_dedup_kernel(const uint8_t* x, const int32_t* __restrict__ idx,
                      const float* __restrict__ gate, int64_t T, int row_bytes, int E, int k,
                      int cpr, const int32_t* gbase, const uint8_t* tcnt,
                      const uint32_t* lslot, int64_t Bp, int64_t G,
                      const int32_t* header, uint8_t* __restrict__ send,
                      int32_t* __restrict__ row_token, int32_t* __restrict__ row_experts,
                      float* __restrict__ row_gates, float* __restrict__ row_weight,
                      int32_t* __restrict__ slot_row, int32_t* __restrict__ n_rows,
                      CoselectBm cs, int cs_blocks, ScanArgs sa) {
  if (coselect_part(cs, cs_blocks)) return;
  const unsigned bid = blockIdx.x - unsigned(cs_blocks), nb = gridDim.x - unsigned(cs_blocks);
  if (!SC && bid == 0 && threadIdx.x == 0) *n_rows = header[0];
  const int lane = lane_id();
  const int jl = lane < k ? lane : k - 1;
  const int64_t wid = (int64_t(bid) * blockDim.x + threadIdx.x) / kWave;
  const int64_t t = wid / cpr;
  const int64_t wm = (meta_block<META>(bid, nb) * blockDim.x + threadIdx.x) / kWave;
  const int64_t tm = wm / cpr;
  const bool copy = t < T;                      // wave-uniform
  const bool meta = tm < T && wm == tm * cpr;   // wave-uniform: one wave per token
  if (!SC && !copy && !meta) return;            // (with SC every wave takes the scan's barriers)
  const int64_t tl = copy ? t : (meta ? tm : T - 1);
  const int64_t tml = meta ? tm : tl;
  const int c = int(wid - t * cpr);
  const int64_t chunk0 = int64_t(c) * (NV * kWave * 16);
  const uint32_t code = lslot[tl * k + jl];  // (rank << 8) | rank inside the tile
  const uint32_t code_m = META ? lslot[tml * k + jl] : code;
  const int e_m = clampi(idx[tml * k + jl], 0, E - 1);
  const float g_m = gate[tml * k + jl];
  ScanPrefetch<sc_vectors(SC)> pf;
  if (SC) {
    scan_prefetch<false>(tcnt, int(G), E, sa.R, sa, pf);
    issue_fence();
  }
  u32x4 v[NV];
  load_chunk<NV>(v, x + tl * row_bytes, chunk0, row_bytes, lane);
  issue_fence();
  int32_t* s_col = nullptr;
  int32_t* s_pre = nullptr;
  if (SC) {
    extern __shared__ uint64_t s_scan[];
    const int total = scan_small_plan<true, false>(tcnt, int(G), sa, pf, bid == 0,
                                                   reinterpret_cast<uint8_t*>(s_scan), s_col,
                                                   s_pre);
    if (bid == 0 && threadIdx.x == 0) *n_rows = total;
    if (!copy && !meta) return;
  }
  const int r_own = int(code >> 8);
  const int pos = (SC ? lds_first_row(s_col, s_pre, tcnt, Bp, G, E + r_own, r_own, tl / kTile)
                      : tile_first_row(gbase, tcnt, Bp, G, E + r_own, r_own, tl / kTile)) +
                  int(code & 255u);
  const int rm_own = int(code_m >> 8);
  const int pos_m =
      META ? (SC ? lds_first_row(s_col, s_pre, tcnt, Bp, G, E + rm_own, rm_own, tml / kTile)
                 : tile_first_row(gbase, tcnt, Bp, G, E + rm_own, rm_own, tml / kTile)) +
                 int(code_m & 255u)
           : pos;
  issue_fence();
  ready(pos_m);
  ready(e_m);
  if (copy) {
    // one row per rank the token is sent to, written by the rank's first slot
    // (the row's leader); lanes >= k match no slot
    const int r = lane < k ? r_own : -1;
    bool leader = lane < k;
    for (int i = 0; i < k; ++i)
      if (i < lane && bcast(r, i) == r) leader = false;
    const uint64_t lm = __ballot(leader);
    for (int j = 0; j < k; ++j) {
      if (!((lm >> j) & 1ull)) continue;
      const int p = bcast(pos, j);
      store_chunk<NV, NT>(v, send + int64_t(p) * row_bytes + chunk0, chunk0, row_bytes, lane);
    }
  }
  if (!meta) return;
  // Metadata of token tm, after the row stores (see the plain kernel).  Per
  // slot: is it the first slot of its rank (the row's leader)?  Its column
  // among the rank's experts (ascending id), the rank's slot count, and its
  // position in the token's ascending expert order.
  const int r = lane < k ? rm_own : -1;
  bool leader = lane < k;
  int col = 0, cnt = 0, sidx = 0;
  for (int i = 0; i < k; ++i) {
    const int ri = bcast(r, i), ei = bcast(e_m, i);
    if (ri == r) {
      ++cnt;
      if (ei < e_m) ++col;
      if (i < lane) leader = false;
    }
    if (ei < e_m) ++sidx;
  }
  if (lane < k) {
    slot_row[tm * k + lane] = pos_m;
    row_experts[int64_t(pos_m) * k + col] = e_m;
    row_gates[int64_t(pos_m) * k + col] = g_m;
    if (leader) {
      row_token[pos_m] = int32_t(tm);
      for (int cc = cnt; cc < k; ++cc) {
        row_experts[int64_t(pos_m) * k + cc] = -1;
        row_gates[int64_t(pos_m) * k + cc] = 0.0f;
      }
    }
  }
  // row weight: fp64 sum of the rank's gates in ascending expert order
  double wsum = 0.0;
  for (int s = 0; s < k; ++s) {
    const uint64_t sm = __ballot(lane < k && sidx == s);
    if (sm == 0ull) continue;  // only if topk_idx repeats an expert (precondition)
    const int src = __ffsll((unsigned long long)sm) - 1;
    const float gs = bcastf(g_m, src);
    const int rs = bcast(r, src);
    if (leader && rs == r) wsum += double(gs);
  }
  if (leader) row_weight[pos_m] = float(wsum);
}

#ifndef MOE_DISPATCH_NT
#define MOE_DISPATCH_NT 0
#endif

constexpr int64_t kMetaMinBlocks = 512;

// Vectors of 16 B per lane per wave: a 4 KiB chunk per wave for long rows.
static int dispatch_nv(int row_bytes) {
  const int vr = row_bytes / 16;
  if (vr >= 4 * kWave) return 4;
  if (vr >= 2 * kWave) return 2;
  return 1;
}

template <int NV>
static hipError_t launch_dispatch_nv(const void* x, const int32_t* idx, const float* gate,
                                     int64_t T, int row_bytes, int E, int k, int R,
                                     const void* workspace, int dedup,
                                     void* send, int32_t* row_token, int32_t* row_e,
                                     float* row_gates, float* row_weight, int32_t* slot_row,
                                     int32_t* n_rows, int64_t cs_tokens, int32_t* W,
                                     const ScanArgs* scan, hipStream_t stream) {
  const PlanLayout pl = plan_layout(T, E, k, R, dedup);
  const uint8_t* ws = static_cast<const uint8_t*>(workspace);
  const int32_t* header = reinterpret_cast<const int32_t*>(ws);
  const int32_t* gbase = reinterpret_cast<const int32_t*>(ws + pl.base_off);
  const uint8_t* tcnt = ws + pl.tcnt_off;
  const uint32_t* lslot = reinterpret_cast<const uint32_t*>(ws + pl.lslot_off);
  CoselectBm cs{};
  int csb = 0;  // co-selection blocks in front of the copy blocks
  size_t lds = 0;
  if (W != nullptr && cs_tokens > 0) {
    cs = coselect_bm_args(reinterpret_cast<const uint64_t*>(ws + pl.bm_off), cs_tokens, E, W);
    csb = int((cs.blocks() + 7) & ~int64_t(7));
    lds = kBmLdsBytes;
  }
  // the plan scanned by the dispatch workgroups themselves (small plans)
  ScanArgs sa{};
  int sc = 0;
  if (scan != nullptr) {
    sa = *scan;
    const bool ranked = !dedup && sa.place != nullptr;
    const bool wide = int64_t(pl.pos_cols) * pl.groups > 4 * 256;
    sc = (ranked ? 2 : 1) + (wide ? 2 : 0);
    const int G = int(pl.groups);
    const size_t sl = ranked ? scan_lds_bytes<true>(pl.cols, pl.pos_cols, E, G)
                             : scan_lds_bytes<false>(pl.cols, pl.pos_cols, E, G);
    lds = lds > sl ? lds : sl;
  }
  const int chunk = NV * kWave * 16;
  const int cpr = (row_bytes + chunk - 1) / chunk;
  const int64_t waves = T * cpr;
  int64_t blocks = (waves + 3) / 4;
  if (blocks == 0) blocks = 1;  // dedup still reports n_rows
  // the XCD-contiguous metadata order from 512 blocks on (2 per CU: below that
  // the waves wait on latency, not bandwidth), on a grid of a multiple of 8
  const bool meta = blocks >= kMetaMinBlocks;
  if (meta) blocks = (blocks + 7) & ~int64_t(7);
  constexpr bool NT = MOE_DISPATCH_NT != 0;
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  uint8_t* sb = static_cast<uint8_t*>(send);
  const dim3 grid{unsigned(blocks + csb)}, block{256};
#define MOE_DISPATCH(META, SC)                                                                 \
  hipLaunchKernelGGL((dispatch_kernel<NV, NT, false, META, SC>), grid, block, lds, stream, xb,  \
                     gate, T, row_bytes, k, cpr, gbase, tcnt, lslot, pl.tiles_pad, pl.groups,  \
                     sb, row_token, row_e, row_weight, slot_row, nullptr, int64_t(0), cs, csb, \
                     sa)
#define MOE_DISPATCH_DEDUP(META, SC)                                                            \
  hipLaunchKernelGGL((dispatch_dedup_kernel<NV, NT, META, SC>), grid, block, lds, stream, xb,   \
                     idx, gate, T, row_bytes, E, k, cpr, gbase, tcnt, lslot, pl.tiles_pad,      \
                     pl.groups, header, sb, row_token, row_e, row_gates, row_weight, slot_row,  \
                     n_rows, cs, csb, sa)
  if (!dedup) {
    if (T == 0) return hipSuccess;
    switch (sc * 2 + (meta ? 1 : 0)) {
      case 0: MOE_DISPATCH(false, 0); break;
      case 1: MOE_DISPATCH(true, 0); break;
      case 2: MOE_DISPATCH(false, 1); break;
      case 3: MOE_DISPATCH(true, 1); break;
      case 4: MOE_DISPATCH(false, 2); break;
      case 5: MOE_DISPATCH(true, 2); break;
      case 6: MOE_DISPATCH(false, 3); break;
      case 7: MOE_DISPATCH(true, 3); break;
      case 8: MOE_DISPATCH(false, 4); break;
      default: MOE_DISPATCH(true, 4); break;
    }
  } else {
    switch (sc * 2 + (meta ? 1 : 0)) {  // sc is 0, 1 or 3 (never ranked)
      case 0: MOE_DISPATCH_DEDUP(false, 0); break;
      case 1: MOE_DISPATCH_DEDUP(true, 0); break;
      case 2: MOE_DISPATCH_DEDUP(false, 1); break;
      case 3: MOE_DISPATCH_DEDUP(true, 1); break;
      case 6: MOE_DISPATCH_DEDUP(false, 3); break;
      default: MOE_DISPATCH_DEDUP(true, 3); break;
    }
  }
#undef MOE_DISPATCH
#undef MOE_DISPATCH_DEDUP
  return hipGetLastError();
}

static hipError_t launch_dispatch_any(const void* x, const int32_t* idx, const float* gate,
                                      int64_t T, int row_bytes, int E, int k, int R,
                                      const void* workspace, int dedup, void* send,
                                      int32_t* row_token, int32_t* row_e, float* row_gates,
                                      float* row_weight, int32_t* slot_row, int32_t* n_rows,
                                      int64_t cs_tokens, int32_t* W, const ScanArgs* scan,
                                      hipStream_t stream) {
  switch (dispatch_nv(row_bytes)) {
    case 4:
      return launch_dispatch_nv<4>(x, idx, gate, T, row_bytes, E, k, R, workspace, dedup,
                                   send, row_token, row_e, row_gates, row_weight, slot_row,
                                   n_rows, cs_tokens, W, scan, stream);
    case 2:
      return launch_dispatch_nv<2>(x, idx, gate, T, row_bytes, E, k, R, workspace, dedup,
                                   send, row_token, row_e, row_gates, row_weight, slot_row,
                                   n_rows, cs_tokens, W, scan, stream);
    default:
      return launch_dispatch_nv<1>(x, idx, gate, T, row_bytes, E, k, R, workspace, dedup,
                                   send, row_token, row_e, row_gates, row_weight, slot_row,
                                   n_rows, cs_tokens, W, scan, stream);
  }
}

// W non-null (and cs_tokens > 0): also the co-selection counts of the first
// cs_tokens tokens, from the plan's expert bitmaps, in the same launch.
hipError_t launch_dispatch(const void* x, const int32_t* idx, const float* gate, int64_t T,
                           int row_bytes, int E, int k, int R, const void* workspace, int dedup,
                           void* send, int32_t* row_token,
                           int32_t* row_e, float* row_gates, float* row_weight,
                           int32_t* slot_row, int32_t* n_rows, int64_t cs_tokens, int32_t* W,
                           hipStream_t stream) {
  return launch_dispatch_any(x, idx, gate, T, row_bytes, E, k, R, workspace, dedup, send,
                             row_token, row_e, row_gates, row_weight, slot_row, n_rows,
                             cs_tokens, W, nullptr, stream);
}

// Copy workgroups of a dispatch of T rows of row_bytes (before padding the
// grid to a multiple of 8): four waves, each one row chunk.
static int64_t dispatch_copy_blocks(int64_t T, int row_bytes) {
  const int chunk = dispatch_nv(row_bytes) * kWave * 16;
  const int64_t cpr = (row_bytes + chunk - 1) / chunk;
  return (T * cpr + 3) / 4;
}

// Whether the dispatch workgroups (256 threads) scan this plan themselves: at
// most kEmbedMaxVec tile-count vectors of position columns (eight per thread),
// at most kEmbedMaxVecBlocks of them over all copy workgroups, and E and R at
// most 256 for the column order and the counts.
bool dispatch_scans_plan(int64_t T, int E, int k, int R, int dedup, int row_bytes) {
  const PlanLayout pl = plan_layout(T, E, k, R, dedup);
  const int64_t nvec = int64_t(pl.pos_cols) * pl.groups;
  return T > 0 && E <= 256 && R <= 256 && nvec <= kEmbedMaxVec &&
         nvec * dispatch_copy_blocks(T, row_bytes) <= kEmbedMaxVecBlocks;
}

// The dispatch of a plan whose tile counts, slot codes and bitmaps the fused
// routing kernel has just written (no scan yet): the dispatch workgroups scan
// it, and workgroup 0 writes the counts, offsets, header and group bases.
// Only for plans that dispatch_scans_plan() accepts.
hipError_t launch_dispatch_scan(const void* x, const int32_t* idx, const float* gate, int64_t T,
                                int row_bytes, int E, int k, int R, const int32_t* place,
                                void* workspace, int dedup, void* send, int32_t* row_token,
                                int32_t* row_e, float* row_gates, float* row_weight,
                                int32_t* slot_row, int32_t* n_rows, int32_t* expert_counts,
                                int32_t* rank_counts, int32_t* rank_offsets,
                                int32_t* expert_offsets, int64_t cs_tokens, int32_t* W,
                                hipStream_t stream) {
  const PlanLayout pl = plan_layout(T, E, k, R, dedup);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  ScanArgs sa;
  sa.B = int(pl.tiles);
  sa.E = E;
  sa.R = R;
  sa.m = E / R;
  sa.place = dedup ? nullptr : place;
  sa.expert_counts = expert_counts;
  sa.rank_counts = rank_counts;
  sa.rank_offsets = rank_offsets;
  sa.expert_offsets = dedup ? nullptr : expert_offsets;
  sa.header = reinterpret_cast<int32_t*>(ws);
  sa.gbase = reinterpret_cast<int32_t*>(ws + pl.base_off);
  return launch_dispatch_any(x, idx, gate, T, row_bytes, E, k, R, workspace, dedup, send,
                             row_token, row_e, row_gates, row_weight, slot_row, n_rows,
                             cs_tokens, W, &sa, stream);
}


template <int NV>
static hipError_t launch_expand_nv(const void* rows, const float* row_gates,
                                   const int32_t* n_rows, int64_t cap, int row_bytes, int E,
                                   int k, int R, const void* workspace, void* expanded,
                                   int64_t out_cap, int32_t* exp_row, int32_t* exp_expert,
                                   float* exp_gate, int32_t* row_slot, hipStream_t stream) {
  const PlanLayout pl = plan_layout(cap, E, k, R, 0);
  const uint8_t* ws = static_cast<const uint8_t*>(workspace);
  const int32_t* gbase = reinterpret_cast<const int32_t*>(ws + pl.base_off);
  const uint8_t* tcnt = ws + pl.tcnt_off;
  const uint32_t* lslot = reinterpret_cast<const uint32_t*>(ws + pl.lslot_off);
  const int chunk = NV * kWave * 16;
  const int cpr = (row_bytes + chunk - 1) / chunk;
  const int64_t blocks = (cap * cpr + 3) / 4;
  constexpr bool NT = MOE_DISPATCH_NT != 0;
  hipLaunchKernelGGL((dispatch_kernel<NV, NT, true, false, 0>), dim3(unsigned(blocks)), dim3(256),
                     0, stream, static_cast<const uint8_t*>(rows), row_gates, cap, row_bytes, k, cpr,
                     gbase, tcnt, lslot, pl.tiles_pad, pl.groups,
                     static_cast<uint8_t*>(expanded), exp_row, exp_expert, exp_gate, row_slot,
                     n_rows, out_cap, CoselectBm{}, 0, ScanArgs{});
  return hipGetLastError();
}

hipError_t launch_expand(const void* rows, const float* row_gates, const int32_t* n_rows,
                         int64_t cap, int row_bytes, int E, int k, int R, const void* workspace,
                         void* expanded, int64_t out_cap, int32_t* exp_row, int32_t* exp_expert,
                         float* exp_gate, int32_t* row_slot, hipStream_t stream) {
  if (cap == 0) return hipSuccess;
  switch (dispatch_nv(row_bytes)) {
    case 4:
      return launch_expand_nv<4>(rows, row_gates, n_rows, cap, row_bytes, E, k, R, workspace,
                                 expanded, out_cap, exp_row, exp_expert, exp_gate, row_slot,
                                 stream);
    case 2:
      return launch_expand_nv<2>(rows, row_gates, n_rows, cap, row_bytes, E, k, R, workspace,
                                 expanded, out_cap, exp_row, exp_expert, exp_gate, row_slot,
                                 stream);
    default:
      return launch_expand_nv<1>(rows, row_gates, n_rows, cap, row_bytes, E, k, R, workspace,
                                 expanded, out_cap, exp_row, exp_expert, exp_gate, row_slot,
                                 stream);
  }
}

}  // namespace moe
