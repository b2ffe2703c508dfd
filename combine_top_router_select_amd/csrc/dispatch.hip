// A4a / A4b - dispatch permute into a rank-contiguous send buffer.
//
// Source: "Expert Coupling in MoE Pretraining" (summary), "Method 1: Correlated
// Expert Placement + Deduplicating Dispatcher": the conventional dispatcher
// sends one copy of a token's hidden state per (token, expert); the
// deduplicating one sends one row per distinct (token, destination rank) with
// the ids and routing probabilities of the rank's selected experts as
// metadata.  "DODOCO" dataset card, "Reading the counts": a token routed to
// several experts on one rank is counted (and sent) once per expert by the
// conventional dispatcher.
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
template <bool META>
__device__ __forceinline__ int64_t meta_block() {
  if (!META) return blockIdx.x;
  const unsigned per = gridDim.x >> 3;
  return int64_t(blockIdx.x & 7u) * per + (blockIdx.x >> 3);
}

// PAD: the receive-side expansion, where a "token" is a received row, slots
// with the code kNoSlot are empty, only rows below *n_valid are expanded, and
// no row is written at or past out_cap (such slots get slot_row = -1).
//
// Each wave copies the row chunk of (token t, chunk c) and writes the metadata
// of token tm (when its wave index in the metadata order is chunk 0 of tm).
// Every load of both is issued before the first wait, from in-bounds indices.
template <int NV, bool NT, bool PAD, bool META>
__global__ void __launch_bounds__(256)
dispatch_kernel(const uint8_t* x, const float* __restrict__ gate, int64_t T,
                int row_bytes, int k, int cpr, const int32_t* gbase,
                const uint8_t* tcnt, const uint32_t* lslot, int64_t Bp,
                int64_t G, uint8_t* __restrict__ send,
                int32_t* __restrict__ row_token, int32_t* __restrict__ row_expert,
                float* __restrict__ row_weight, int32_t* __restrict__ slot_row,
                const int32_t* __restrict__ n_valid, int64_t out_cap) {
  const int lane = lane_id();
  // lanes j < k own slot j; the other lanes load slot k-1's data and ignore it
  const int jl = lane < k ? lane : k - 1;
  const int64_t nv = PAD ? int64_t(*n_valid) : T;
  const int64_t wid = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;
  const int64_t t = wid / cpr;
  const int64_t wm = (meta_block<META>() * blockDim.x + threadIdx.x) / kWave;
  const int64_t tm = wm / cpr;
  static_assert(!(PAD && META), "the expansion writes the metadata of its own rows");
  const int c = int(wid - t * cpr);
  if (PAD && t < T && t >= nv) {  // whole wave: a row past the received ones
    if (c == 0 && lane < k) slot_row[t * k + lane] = -1;
    return;
  }
  const bool copy = t < T && t < nv;            // wave-uniform
  const bool meta = tm < T && wm == tm * cpr;   // wave-uniform: one wave per token
  if (!copy && !meta) return;
  // The loads are unconditional, from tokens in range: a load under a branch
  // the compiler cannot prove uniform is followed by a wait for it.
  const int64_t tl = copy ? t : tm;
  const int64_t tml = meta ? tm : t;
  const int64_t chunk0 = int64_t(c) * (NV * kWave * 16);
  const uint32_t code = lslot[tl * k + jl];  // (expert << 8) | rank inside the tile
  const uint32_t code_m = META ? lslot[tml * k + jl] : code;
  const float g_m = gate[tml * k + jl];
  u32x4 v[NV];
  load_chunk<NV>(v, x + tl * row_bytes, chunk0, row_bytes, lane);
  issue_fence();
  const bool has = !PAD || code != kNoSlot;
  const int e = has ? int(code >> 8) : 0;
  const int pos = tile_first_row(gbase, tcnt, Bp, G, e, e, tl / kTile) + int(code & 255u);
  const bool has_m = !PAD || code_m != kNoSlot;
  const int e_m = has_m ? int(code_m >> 8) : 0;
  const int pos_m =
      META ? tile_first_row(gbase, tcnt, Bp, G, e_m, e_m, tml / kTile) + int(code_m & 255u)
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

template <int NV, bool NT, bool META>
__global__ void __launch_bounds__(256)
dispatch_dedup_kernel(const uint8_t* x, const int32_t* __restrict__ idx,
                      const float* __restrict__ gate, int64_t T, int row_bytes, int E, int k,
                      int cpr, const int32_t* gbase, const uint8_t* tcnt,
                      const uint32_t* lslot, int64_t Bp, int64_t G,
                      const int32_t* __restrict__ header, uint8_t* __restrict__ send,
                      int32_t* __restrict__ row_token, int32_t* __restrict__ row_experts,
                      float* __restrict__ row_gates, float* __restrict__ row_weight,
                      int32_t* __restrict__ slot_row, int32_t* __restrict__ n_rows) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_rows = header[0];
  const int lane = lane_id();
  const int jl = lane < k ? lane : k - 1;
  const int64_t wid = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;
  const int64_t t = wid / cpr;
  const int64_t wm = (meta_block<META>() * blockDim.x + threadIdx.x) / kWave;
  const int64_t tm = wm / cpr;
  const bool copy = t < T;                      // wave-uniform
  const bool meta = tm < T && wm == tm * cpr;   // wave-uniform: one wave per token
  if (!copy && !meta) return;
  const int64_t tl = copy ? t : tm;
  const int64_t tml = meta ? tm : t;
  const int c = int(wid - t * cpr);
  const int64_t chunk0 = int64_t(c) * (NV * kWave * 16);
  const uint32_t code = lslot[tl * k + jl];  // (rank << 8) | rank inside the tile
  const uint32_t code_m = META ? lslot[tml * k + jl] : code;
  const int e_m = clampi(idx[tml * k + jl], 0, E - 1);
  const float g_m = gate[tml * k + jl];
  u32x4 v[NV];
  load_chunk<NV>(v, x + tl * row_bytes, chunk0, row_bytes, lane);
  issue_fence();
  const int r_own = int(code >> 8);
  const int pos = tile_first_row(gbase, tcnt, Bp, G, E + r_own, r_own, tl / kTile) +
                  int(code & 255u);
  const int rm_own = int(code_m >> 8);
  const int pos_m =
      META ? tile_first_row(gbase, tcnt, Bp, G, E + rm_own, rm_own, tml / kTile) +
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
                                     int32_t* n_rows, hipStream_t stream) {
  const PlanLayout pl = plan_layout(T, E, k, R, dedup);
  const uint8_t* ws = static_cast<const uint8_t*>(workspace);
  const int32_t* header = reinterpret_cast<const int32_t*>(ws);
  const int32_t* gbase = reinterpret_cast<const int32_t*>(ws + pl.base_off);
  const uint8_t* tcnt = ws + pl.tcnt_off;
  const uint32_t* lslot = reinterpret_cast<const uint32_t*>(ws + pl.lslot_off);
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
  const dim3 grid{unsigned(blocks)}, block{256};
  if (!dedup) {
    if (T == 0) return hipSuccess;
    if (meta)
      hipLaunchKernelGGL((dispatch_kernel<NV, NT, false, true>), grid, block, 0, stream, xb, gate,
                         T, row_bytes, k, cpr, gbase, tcnt, lslot, pl.tiles_pad, pl.groups, sb,
                         row_token, row_e, row_weight, slot_row, nullptr, int64_t(0));
    else
      hipLaunchKernelGGL((dispatch_kernel<NV, NT, false, false>), grid, block, 0, stream, xb,
                         gate, T, row_bytes, k, cpr, gbase, tcnt, lslot, pl.tiles_pad, pl.groups,
                         sb, row_token, row_e, row_weight, slot_row, nullptr, int64_t(0));
  } else {
    if (meta)
      hipLaunchKernelGGL((dispatch_dedup_kernel<NV, NT, true>), grid, block, 0, stream, xb, idx,
                         gate, T, row_bytes, E, k, cpr, gbase, tcnt, lslot, pl.tiles_pad,
                         pl.groups, header, sb, row_token, row_e, row_gates, row_weight,
                         slot_row, n_rows);
    else
      hipLaunchKernelGGL((dispatch_dedup_kernel<NV, NT, false>), grid, block, 0, stream, xb, idx,
                         gate, T, row_bytes, E, k, cpr, gbase, tcnt, lslot, pl.tiles_pad,
                         pl.groups, header, sb, row_token, row_e, row_gates, row_weight,
                         slot_row, n_rows);
  }
  return hipGetLastError();
}

hipError_t launch_dispatch(const void* x, const int32_t* idx, const float* gate, int64_t T,
                           int row_bytes, int E, int k, int R, const void* workspace, int dedup,
                           void* send, int32_t* row_token,
                           int32_t* row_e, float* row_gates, float* row_weight,
                           int32_t* slot_row, int32_t* n_rows, hipStream_t stream) {
  switch (dispatch_nv(row_bytes)) {
    case 4:
      return launch_dispatch_nv<4>(x, idx, gate, T, row_bytes, E, k, R, workspace, dedup,
                                   send, row_token, row_e, row_gates, row_weight, slot_row,
                                   n_rows, stream);
    case 2:
      return launch_dispatch_nv<2>(x, idx, gate, T, row_bytes, E, k, R, workspace, dedup,
                                   send, row_token, row_e, row_gates, row_weight, slot_row,
                                   n_rows, stream);
    default:
      return launch_dispatch_nv<1>(x, idx, gate, T, row_bytes, E, k, R, workspace, dedup,
                                   send, row_token, row_e, row_gates, row_weight, slot_row,
                                   n_rows, stream);
  }
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
  hipLaunchKernelGGL((dispatch_kernel<NV, NT, true, false>), dim3(unsigned(blocks)), dim3(256), 0,
                     stream, static_cast<const uint8_t*>(rows), row_gates, cap, row_bytes, k, cpr,
                     gbase, tcnt, lslot, pl.tiles_pad, pl.groups,
                     static_cast<uint8_t*>(expanded), exp_row, exp_expert, exp_gate, row_slot,
                     n_rows, out_cap);
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
