// A2 + A3 - send counts, exclusive scan, and the per-tile plan used by dispatch.
//
// Sources: "DODOCO: MoE AlltoAll Traffic Matrices on Real Text" (dataset card),
// sections "Setup" (the counts are the dispatcher's per-destination input
// splits; contiguous placement) and "Reading the counts" (one count per
// token-expert assignment; rows sum to tokens x top-k; each rank's expert block
// sums to its receive total).  "Expert Coupling in MoE Pretraining" (summary),
// "Method 1": the deduplicating dispatcher sends one row per distinct
// (token, destination rank).
//
// Counting 64 tokens (one wave, one lane per token), i.e. 64 / kTile plan
// tiles: every column (expert; in dedup mode also rank) gets a 64-bit LDS
// bitmap of the tokens that use it, built with ds_or_b64 (order independent).
// popcount of the bits of a lane's own tile below the lane is the token's rank
// among its tile's earlier users of the column; popcount of a tile's bits is
// its count.  The tile counts are then scanned over tiles,
// per column, into the absolute first row of each tile in each column.  A
// row's position is the first row of the tile's 16-tile group in its column
// (written by the scan) + the counts of the group's earlier tiles (summed by
// the dispatch kernel) + rank, which makes the send buffer order
// (rank, expert, token) - or (rank, token) - stable and deterministic.  No
// global atomics anywhere.
//
// Two kernels: tile_counts (one wave per 64 tokens, so the per-assignment work
// and its memory traffic spread over many CUs) and plan_scan (one workgroup,
// which only reads the per-tile counts, one byte each, and writes the bases).
// Both per-tile arrays are column-major, so a scan thread streams a run of one
// column's tiles with 16-byte loads and stores.
//
// All global loads are issued unconditionally from clamped, in-bounds
// addresses and only stores are predicated: a load under a branch is followed
// by a wait for it, which would serialise them.
#include "common.hpp"
#include "moe_route.h"
#include "plan_order.hpp"

namespace moe {

// floor(f / k) for 0 <= f < 2^24 and 2 <= k <= 16 is __umulhi(f, ceil(2^32 / k)):
// the rounding error of the reciprocal, below f / 2^32, never reaches 1/k.
__host__ __device__ inline uint32_t kdiv_mul(int k) {
  return k <= 1 ? 0u : uint32_t(((1ull << 32) + uint64_t(k) - 1) / uint64_t(k));
}
__device__ __forceinline__ int kdiv(uint32_t f, uint32_t mul, int k) {
  return k == 1 ? int(f) : int(__umulhi(f, mul));
}

// Raw ids of one tile for the calling wave: lane l takes the tile's flat id
// positions l, l + 64, ... (each load covers 256 contiguous bytes).  Positions
// past the end read the last id instead (no branch, no out-of-bounds access);
// callers clamp values where they use them, so that a prefetch does not wait
// for its own loads.
template <int KMAX>
__device__ __forceinline__ void load_tile_ids(int (&raw)[KMAX], const int32_t* __restrict__ idx,
                                              int64_t f0, int64_t total, int lane) {
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    const int64_t f = f0 + lane + kWave * r;
    raw[r] = idx[f < total ? f : total - 1];
  }
}

// Counts 64 tokens (four plan tiles) in the calling wave.  `bits` holds C
// zeroed bitmaps: column c's bit i is set when token i of the 64 uses column c.
// Lane l owns the ids at flat positions l + 64 r of the block (token
// (l + 64 r) / k, slot (l + 64 r) % k) and writes their slot codes back at the
// same positions, so loads and stores stay coalesced.  A slot's rank counts the
// earlier tokens of its own plan tile only.  In dedup mode every id also
// sets its token's bit in its rank's bitmap (setting it twice is harmless).
// `s_rank` maps expert -> rank (LDS) or is null for contiguous placement.
// PAD (received rows): negative ids are empty slots and only the first
// `tvalid` rows of the tile are counted; empty entries get the code kNoSlot.
template <bool DEDUP, bool PAD, int KMAX>
__device__ __forceinline__ void count_tile(const int (&raw)[KMAX], int64_t f0, int nf, int k,
                                           uint32_t kmul, int E, const int32_t* s_rank, int m,
                                           int tvalid, uint64_t* bits,
                                           uint32_t* __restrict__ lslot, int lane) {
  int e[KMAX], col[KMAX], tl[KMAX];
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    const int f = lane + kWave * r;
    e[r] = clampi(raw[r], 0, E - 1);
    tl[r] = kdiv(uint32_t(f), kmul, k);
    tl[r] = tl[r] < kWaveTile ? tl[r] : kWaveTile - 1;  // positions past the block are unused
    col[r] = DEDUP ? (s_rank ? s_rank[e[r]] : e[r] / m) : e[r];
  }
  bool ok[KMAX];
#pragma unroll
  for (int r = 0; r < KMAX; ++r)
    ok[r] = lane + kWave * r < nf && (!PAD || (raw[r] >= 0 && tl[r] < tvalid));
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    if (ok[r]) {
      const unsigned long long bit = 1ull << tl[r];
      atomicOr(reinterpret_cast<unsigned long long*>(&bits[e[r]]), bit);
      if (DEDUP) atomicOr(reinterpret_cast<unsigned long long*>(&bits[E + col[r]]), bit);
    }
  }
  wave_lds_sync();
  uint32_t code[KMAX];
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    const uint64_t mb = bits[DEDUP ? E + col[r] : col[r]];
    const int t0 = tl[r] & ~(kTile - 1);  // first token of the slot's plan tile
    const uint64_t below = ((1ull << tl[r]) - 1ull) & ~((1ull << t0) - 1ull);
    code[r] = (uint32_t(col[r]) << 8) | uint32_t(__popcll(mb & below));
    if (PAD && !ok[r]) code[r] = kNoSlot;
  }
#pragma unroll
  for (int r = 0; r < KMAX; ++r)
    if (lane + kWave * r < nf) lslot[f0 + lane + kWave * r] = code[r];
}

// ----------------------------------------------------------- tile counts --

template <bool DEDUP, bool PAD, int KMAX>
__global__ void __launch_bounds__(kWave)
tile_counts_kernel(const int32_t* __restrict__ idx, int64_t T, int E, int k, int R,
                   const int32_t* __restrict__ place, int m, uint32_t kmul, int64_t Bp,
                   const int32_t* __restrict__ n_valid, uint8_t* __restrict__ tcnt,
                   uint32_t* __restrict__ lslot, uint64_t* __restrict__ bm) {
  extern __shared__ uint64_t s_tdyn[];
  const int C = E + (DEDUP ? R : 0);
  uint64_t* bits = s_tdyn;                                        // [C]
  int32_t* s_rank = reinterpret_cast<int32_t*>(s_tdyn + C);      // [E] (dedup, explicit placement)
  const int lane = lane_id();
  const int64_t b = blockIdx.x;  // 64-token block: plan tiles kTilesPerWave b + 0, 1, ...
  const int64_t f0 = b * kWaveTile * k;
  const int64_t total = T * k;
  const int nf =
      int(total - f0 < int64_t(kWaveTile) * k ? total - f0 : int64_t(kWaveTile) * k);
  int raw[KMAX];
  load_tile_ids<KMAX>(raw, idx, f0, total, lane);
  int tvalid = kWaveTile;  // rows of this block that count (PAD: rows below *n_valid)
  if (PAD) {
    const int64_t nv = *n_valid - b * kWaveTile;
    tvalid = int(nv < 0 ? 0 : (nv > kWaveTile ? kWaveTile : nv));
  }
  for (int c = lane; c < C; c += kWave) bits[c] = 0ull;
  const bool has_rank = DEDUP && place;
  if (has_rank)
    for (int e = lane; e < E; e += kWave) s_rank[e] = clampi(place[e], 0, R - 1);
  wave_lds_sync();
  count_tile<DEDUP, PAD, KMAX>(raw, f0, nf, k, kmul, E, has_rank ? s_rank : nullptr, m, tvalid,
                               bits, lslot, lane);
  // the block's tiles' counts of a column are kTilesPerWave consecutive bytes
  // (Bp is a multiple of 16, so the last block's stay below Bp); tiles past
  // the last one get zeros
  constexpr uint64_t kTileMask = kTile == 64 ? ~0ull : ((1ull << (kTile % 64)) - 1ull);
  for (int c = lane; c < C; c += kWave) {
    const uint64_t mb = bits[c];
#pragma unroll
    for (int q = 0; q < kTilesPerWave; ++q)
      tcnt[c * Bp + kTilesPerWave * b + q] =
          uint8_t(__popcll((mb >> (q * kTile % 64)) & kTileMask));
  }
  if (bm)  // the block's expert bitmaps, for the co-selection counts
    for (int e = lane; e < E; e += kWave) bm[b * E + e] = bits[e];
}

// ------------------------------------------------------------------- scan --

constexpr int kMaxQ = 16;  // lanes per column (one DPP row at most)
constexpr int kMaxKV = 16; // tile vectors per lane held in registers
constexpr int kBatch = 8;  // vectors loaded together by the looping variant

// One workgroup turns the per-tile counts into the plan's group bases: for
// every position column and every group of 16 tiles (one 16-byte vector of
// tile counts), the first row of that group in the send buffer.
//  A. Column sums.  KV > 0: a column's vectors are dealt round-robin to Q
//     consecutive lanes (lane q takes vectors q, q + Q, ...: each load
//     instruction covers Q x 16 contiguous bytes of the column); per round a
//     segmented DPP scan gives each vector the sum of the column's earlier
//     vectors.  KV = 0 (very large plans): one lane per column, looping.
//  B. The columns in scan order - expert id (plain, contiguous placement),
//     rank (dedup), or (rank, id) for plain dispatch with an explicit
//     placement (RANKED: a counting sort with rank bitmasks) - and one
//     block-wide exclusive scan (DPP wave scans) give each column's first row.
//  C. Group bases = column first row + earlier vectors; counts and offsets.
// No global atomics: the plan is a pure function of the counts.
template <bool DEDUP, bool RANKED, int KV>
__global__ void __launch_bounds__(kScanThreads)
plan_scan_kernel(const uint8_t* __restrict__ tcnt, int B, int Bp, int Q, int E, int R,
                 const int32_t* __restrict__ place, int m, int32_t* __restrict__ expert_counts,
                 int32_t* __restrict__ rank_counts, int32_t* __restrict__ rank_offsets,
                 int32_t* __restrict__ expert_offsets, int32_t* __restrict__ header,
                 int32_t* __restrict__ vbase) {
  __shared__ int32_t s_tot[kMaxCols];           // column totals
  __shared__ int32_t s_colbase[MOE_MAX_EXPERTS];  // first row of each position column
  __shared__ OrderLds<RANKED> s_ord;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int nthreads = blockDim.x;
  const int C = E + (DEDUP ? R : 0);
  const int cbase = DEDUP ? E : 0;  // first position column among the counted ones
  const int nvec = Bp / 16;         // 16-tile vectors per column
  const u32x4* g4 = reinterpret_cast<const u32x4*>(tcnt);

  // A. column sums; the loads go out first
  constexpr int NK = KV > 0 ? KV : 1;
  const int units = C * Q;
  const bool active = KV > 0 && tid < units;
  const int c = tid / Q, q = tid & (Q - 1);
  int pre[NK];
  if (KV > 0) {
    u32x4 v[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int vi = q + Q * i;
      v[i] = g4[size_t(active ? c : 0) * nvec + (vi < nvec ? vi : nvec - 1)];
    }
    int run = 0;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int vi = q + Q * i;
      const int vs = (active && vi < nvec) ? byte_sum(keep_bytes(v[i], B - 16 * vi)) : 0;
      const int incl = segment_incl_scan(vs, Q, lane);
      pre[i] = run + incl - vs;
      run += __shfl(incl, (lane & ~(Q - 1)) + Q - 1, kWave);  // the round's column total
    }
    if (active && q == 0) s_tot[c] = run;
  } else {
    for (int cc = tid; cc < C; cc += nthreads) {
      int sum = 0;
      for (int b0 = 0; b0 < nvec; b0 += kBatch) {
        u32x4 t[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
          t[i] = g4[size_t(cc) * nvec + (b0 + i < nvec ? b0 + i : nvec - 1)];
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
          sum += b0 + i < nvec ? byte_sum(keep_bytes(t[i], B - 16 * (b0 + i))) : 0;
      }
      s_tot[cc] = sum;
    }
  }
  int my_rank = 0;
  if (RANKED && tid < E) my_rank = clampi(place[tid], 0, R - 1);
  order_init<RANKED>(s_ord);
  __syncthreads();

  // B. scan order, the block-wide scan, counts and offsets
  order_columns<DEDUP, RANKED>(s_tot, s_colbase, s_ord, E, R, m, my_rank, true, expert_counts,
                               rank_counts, rank_offsets, expert_offsets, header);

  // C. group bases
  if (KV > 0) {
    if (active && c >= cbase) {
      const int cb = s_colbase[c - cbase];
      int32_t* col = vbase + size_t(c - cbase) * nvec;
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const int vi = q + Q * i;
        if (vi < nvec) col[vi] = cb + pre[i];
      }
    }
  } else {
    for (int cc = cbase + tid; cc < C; cc += nthreads) {
      int run = s_colbase[cc - cbase];
      int32_t* col = vbase + size_t(cc - cbase) * nvec;
      for (int b0 = 0; b0 < nvec; b0 += kBatch) {
        u32x4 t[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
          t[i] = g4[size_t(cc) * nvec + (b0 + i < nvec ? b0 + i : nvec - 1)];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          if (b0 + i < nvec) {
            col[b0 + i] = run;
            run += byte_sum(keep_bytes(t[i], B - 16 * (b0 + i)));
          }
        }
      }
    }
  }
}

// ----------------------------------------------- scan of large plans --
//
// Past kSplitVec vectors (16-tile groups) per column the one-workgroup scan
// runs long (the receive-side plan of 98304 rows: 96 vectors in each of 128
// columns).  There the scan runs as two kernels of many workgroups (measured
// on that plan's 16384-token top-6 receive step: 844.8 -> 842.5 us; at 32
// vectors, the 16384-token top-2 step, one workgroup stays faster, 265.3
// against 266.8 us): the column totals
// (one workgroup per column), then the bases (one workgroup per position
// column): each of those orders the columns and scans their totals itself -
// cheap, in LDS - and scans its own column's vectors; workgroup 0 also writes
// the counts and offsets.  Same plan, bit for bit, still no global atomics.
constexpr int kSplitVec = 32;
constexpr int kColThreads = 256;

// Sum over the workgroup (blockDim.x a multiple of 64, at most 1024); every
// thread gets it.
__device__ __forceinline__ int block_sum(int v, int32_t* s_w) {
  const int lane = lane_id(), w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  const int incl = wave_incl_scan(v);
  __syncthreads();  // s_w may still be read by an earlier call
  if (lane == kWave - 1) s_w[w] = incl;
  __syncthreads();
  int t = 0;
  for (int i = 0; i < nw; ++i) t += s_w[i];
  return t;
}

// Exclusive scan over the workgroup; *total gets the sum.
__device__ __forceinline__ int block_excl_scan(int v, int32_t* s_w, int* total) {
  const int lane = lane_id(), w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  const int incl = wave_incl_scan(v);
  __syncthreads();
  if (lane == kWave - 1) s_w[w] = incl;
  __syncthreads();
  int carry = 0, t = 0;
  for (int i = 0; i < nw; ++i) {
    carry += i < w ? s_w[i] : 0;
    t += s_w[i];
  }
  *total = t;
  return carry + incl - v;
}

// Column c = blockIdx.x: the sum of its tile counts.
__global__ void __launch_bounds__(kColThreads)
plan_colsum_kernel(const uint8_t* __restrict__ tcnt, int B, int Bp,
                   int32_t* __restrict__ ctot) {
  __shared__ int32_t s_w[kColThreads / kWave];
  const int c = blockIdx.x;
  const int nvec = Bp / 16;
  const u32x4* g4 = reinterpret_cast<const u32x4*>(tcnt) + size_t(c) * nvec;
  int sum = 0;
  for (int v0 = 0; v0 < nvec; v0 += 4 * kColThreads) {
    u32x4 t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = v0 + i * kColThreads + int(threadIdx.x);
      t[i] = g4[v < nvec ? v : nvec - 1];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = v0 + i * kColThreads + int(threadIdx.x);
      sum += v < nvec ? byte_sum(keep_bytes(t[i], B - 16 * v)) : 0;
    }
  }
  const int total = block_sum(sum, s_w);
  if (threadIdx.x == 0) ctot[c] = total;
}

// Position column p = blockIdx.x: the first row of each of its 16-tile groups.
template <bool DEDUP, bool RANKED>
__global__ void __launch_bounds__(kScanThreads)
plan_bases_kernel(const uint8_t* __restrict__ tcnt, int B, int Bp, int E, int R,
                  const int32_t* __restrict__ place, int m, const int32_t* __restrict__ ctot,
                  int32_t* __restrict__ expert_counts, int32_t* __restrict__ rank_counts,
                  int32_t* __restrict__ rank_offsets, int32_t* __restrict__ expert_offsets,
                  int32_t* __restrict__ header, int32_t* __restrict__ vbase) {
  __shared__ int32_t s_tot[kMaxCols];
  __shared__ int32_t s_colbase[MOE_MAX_EXPERTS];
  __shared__ OrderLds<RANKED> s_ord;
  __shared__ int32_t s_w[kScanWaves];
  const int tid = threadIdx.x;
  const int p = blockIdx.x;
  const int C = E + (DEDUP ? R : 0);
  const int cbase = DEDUP ? E : 0;
  const int nvec = Bp / 16;
  const u32x4* g4 = reinterpret_cast<const u32x4*>(tcnt) + size_t(cbase + p) * nvec;
  // this column's first vectors go out first
  const u32x4 first = g4[tid < nvec ? tid : nvec - 1];
  for (int c = tid; c < C; c += blockDim.x) s_tot[c] = ctot[c];
  int my_rank = 0;
  if (RANKED && tid < E) my_rank = clampi(place[tid], 0, R - 1);
  order_init<RANKED>(s_ord);
  __syncthreads();
  order_columns<DEDUP, RANKED>(s_tot, s_colbase, s_ord, E, R, m, my_rank, p == 0,
                               expert_counts, rank_counts, rank_offsets, expert_offsets, header);
  int run = s_colbase[p];
  int32_t* col = vbase + size_t(p) * nvec;
  for (int v0 = 0; v0 < nvec; v0 += blockDim.x) {
    const int v = v0 + tid;
    const u32x4 t = v0 == 0 ? first : g4[v < nvec ? v : nvec - 1];
    const int x = v < nvec ? byte_sum(keep_bytes(t, B - 16 * v)) : 0;
    int total;
    const int excl = block_excl_scan(x, s_w, &total);
    if (v < nvec) col[v] = run + excl;
    run += total;
  }
}

// The scan of a plan whose tile counts (tcnt) are already in the workspace:
// launched after tile_counts_kernel, or after the fused routing kernel.
hipError_t launch_plan_scan(int64_t T, int E, int k, int R, const int32_t* place, int dedup,
                            int32_t* expert_counts, int32_t* rank_counts, int32_t* rank_offsets,
                            int32_t* expert_offsets, void* workspace, hipStream_t stream) {
  const PlanLayout pl = plan_layout(T, E, k, R, dedup);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* header = reinterpret_cast<int32_t*>(ws);
  int32_t* vbase = reinterpret_cast<int32_t*>(ws + pl.base_off);
  const uint8_t* tcnt = ws + pl.tcnt_off;
  const int m = E / R;
  const int B = int(pl.tiles);
  const int Bp = int(pl.tiles_pad);
  const int nvec = Bp / 16;
  const int CP = pl.pos_cols;
  const bool ranked = !dedup && place != nullptr;
  if (nvec > kSplitVec) {  // large plan: two kernels of many workgroups
    int32_t* ctot = reinterpret_cast<int32_t*>(ws + pl.ctot_off);
    hipLaunchKernelGGL(plan_colsum_kernel, dim3(unsigned(pl.cols)), dim3(kColThreads), 0, stream,
                       tcnt, B, Bp, ctot);
    // a thread per expert: workgroup 0 writes the expert counts (and, ranked,
    // orders the columns by expert), and E also covers the CP position columns
    // and the R ranks (R divides E)
    const int need = E > kColThreads ? E : kColThreads;
    const int threads = (need + kWave - 1) / kWave * kWave;
#define MOE_BASES(D, RK)                                                                      \
  hipLaunchKernelGGL((plan_bases_kernel<D, RK>), dim3(unsigned(CP)), dim3(threads), 0, stream, \
                     tcnt, B, Bp, E, R, place, m, ctot, expert_counts, rank_counts,            \
                     rank_offsets, expert_offsets, header, vbase)
    if (dedup) MOE_BASES(true, false);
    else if (ranked) MOE_BASES(false, true);
    else MOE_BASES(false, false);
#undef MOE_BASES
    return hipGetLastError();
  }
  // lanes per column: a power of two <= 16 with every column's lanes in one
  // workgroup; then vectors per lane
  int Q = kMaxQ;
  while (Q > 1 && (pl.cols * Q > kScanThreads || Q > nvec)) Q >>= 1;
  const int kv = nvec > 0 ? (nvec + Q - 1) / Q : 1;
  int KV = kv <= 1 ? 1 : kv <= 2 ? 2 : kv <= 4 ? 4 : kv <= 8 ? 8 : kv <= kMaxKV ? 16 : 0;
  if (pl.cols * Q > kScanThreads || nvec == 0) KV = 0;  // no tiles: nothing to load
  if (KV == 0) Q = 1;
  int threads = kScanThreads;
  if (KV > 0) {
    int need = pl.cols * Q;
    need = need > CP ? need : CP;
    if (ranked) need = need > E ? need : E;
    threads = (need + kWave - 1) / kWave * kWave;
  }
#define MOE_SCAN_LAUNCH(D, RK, K)                                                               \
  hipLaunchKernelGGL((plan_scan_kernel<D, RK, K>), dim3(1), dim3(threads), 0, stream, tcnt, B,   \
                     Bp, Q, E, R, place, m, expert_counts, rank_counts, rank_offsets,            \
                     expert_offsets, header, vbase)
#define MOE_SCAN_KV(D, RK)                      \
  switch (KV) {                                 \
    case 0: MOE_SCAN_LAUNCH(D, RK, 0); break;   \
    case 1: MOE_SCAN_LAUNCH(D, RK, 1); break;   \
    case 2: MOE_SCAN_LAUNCH(D, RK, 2); break;   \
    case 4: MOE_SCAN_LAUNCH(D, RK, 4); break;   \
    case 8: MOE_SCAN_LAUNCH(D, RK, 8); break;   \
    default: MOE_SCAN_LAUNCH(D, RK, 16); break; \
  }
  if (dedup) {
    MOE_SCAN_KV(true, false)
  } else if (ranked) {
    MOE_SCAN_KV(false, true)
  } else {
    MOE_SCAN_KV(false, false)
  }
#undef MOE_SCAN_KV
#undef MOE_SCAN_LAUNCH
  return hipGetLastError();
}

template <bool PAD, int KMAX>
static hipError_t launch_counts_k(const int32_t* idx, int64_t T, int E, int k, int R,
                                  const int32_t* place, int dedup, const int32_t* n_valid,
                                  int32_t* expert_counts, int32_t* rank_counts,
                                  int32_t* rank_offsets, int32_t* expert_offsets,
                                  void* workspace, hipStream_t stream, bool scan = true) {
  const PlanLayout pl = plan_layout(T, E, k, R, dedup);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* tcnt = ws + pl.tcnt_off;
  uint32_t* lslot = reinterpret_cast<uint32_t*>(ws + pl.lslot_off);
  uint64_t* bm = PAD ? nullptr : reinterpret_cast<uint64_t*>(ws + pl.bm_off);
  const int m = E / R;
  if (T > 0) {
    const size_t lds = size_t(pl.cols) * sizeof(uint64_t) + size_t(E) * sizeof(int32_t);
    const uint32_t kmul = kdiv_mul(k);
    if (dedup)
      hipLaunchKernelGGL((tile_counts_kernel<true, false, KMAX>), dim3(unsigned(pl.bm_tiles)),
                         dim3(kWave), lds, stream, idx, T, E, k, R, place, m, kmul, pl.tiles_pad,
                         n_valid, tcnt, lslot, bm);
    else
      hipLaunchKernelGGL((tile_counts_kernel<false, PAD, KMAX>), dim3(unsigned(pl.bm_tiles)),
                         dim3(kWave), lds, stream, idx, T, E, k, R, place, m, kmul, pl.tiles_pad,
                         n_valid, tcnt, lslot, bm);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (!scan) return hipSuccess;
  return launch_plan_scan(T, E, k, R, place, dedup, expert_counts, rank_counts, rank_offsets,
                          expert_offsets, workspace, stream);
}

hipError_t launch_send_counts(const int32_t* idx, int64_t T, int E, int k, int R,
                              const int32_t* place, int dedup, int32_t* expert_counts,
                              int32_t* rank_counts, int32_t* rank_offsets,
                              int32_t* expert_offsets, void* workspace, hipStream_t stream) {
  if (k <= 2)
    return launch_counts_k<false, 2>(idx, T, E, k, R, place, dedup, nullptr, expert_counts,
                                     rank_counts, rank_offsets, expert_offsets, workspace,
                                     stream);
  if (k <= 4)
    return launch_counts_k<false, 4>(idx, T, E, k, R, place, dedup, nullptr, expert_counts,
                                     rank_counts, rank_offsets, expert_offsets, workspace,
                                     stream);
  if (k <= 8)
    return launch_counts_k<false, 8>(idx, T, E, k, R, place, dedup, nullptr, expert_counts,
                                     rank_counts, rank_offsets, expert_offsets, workspace,
                                     stream);
  return launch_counts_k<false, 16>(idx, T, E, k, R, place, dedup, nullptr, expert_counts,
                                    rank_counts, rank_offsets, expert_offsets, workspace, stream);
}

// The tile counts, slot codes and expert bitmaps of the plan of topk_idx,
// without its scan: the same workspace state as the fused routing kernel
// leaves (for a dispatch that scans the plan later).
hipError_t launch_tile_counts(const int32_t* idx, int64_t T, int E, int k, int R,
                              const int32_t* place, int dedup, void* workspace,
                              hipStream_t stream) {
#define MOE_TC(KM)                                                                           \
  launch_counts_k<false, KM>(idx, T, E, k, R, place, dedup, nullptr, nullptr, nullptr,       \
                             nullptr, nullptr, workspace, stream, false)
  if (k <= 2) return MOE_TC(2);
  if (k <= 4) return MOE_TC(4);
  if (k <= 8) return MOE_TC(8);
  return MOE_TC(16);
#undef MOE_TC
}

// Receive side: the plan of the per-expert expansion of `cap` received rows, of
// which the first *n_rows count; negative ids are empty slots.  Same plan as
// the plain dispatch (rows play the part of tokens).
hipError_t launch_expand_counts(const int32_t* row_experts, int64_t cap, int E, int k, int R,
                                const int32_t* place, const int32_t* n_rows,
                                int32_t* expert_counts, int32_t* rank_counts,
                                int32_t* rank_offsets, int32_t* expert_offsets, void* workspace,
                                hipStream_t stream) {
  if (k <= 2)
    return launch_counts_k<true, 2>(row_experts, cap, E, k, R, place, 0, n_rows, expert_counts,
                                    rank_counts, rank_offsets, expert_offsets, workspace,
                                    stream);
  if (k <= 4)
    return launch_counts_k<true, 4>(row_experts, cap, E, k, R, place, 0, n_rows, expert_counts,
                                    rank_counts, rank_offsets, expert_offsets, workspace,
                                    stream);
  if (k <= 8)
    return launch_counts_k<true, 8>(row_experts, cap, E, k, R, place, 0, n_rows, expert_counts,
                                    rank_counts, rank_offsets, expert_offsets, workspace,
                                    stream);
  return launch_counts_k<true, 16>(row_experts, cap, E, k, R, place, 0, n_rows, expert_counts,
                                   rank_counts, rank_offsets, expert_offsets, workspace, stream);
}

}  // namespace moe
