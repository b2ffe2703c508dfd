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
// Counting a 64-token tile (one wave, one lane per token): every column
// (expert; in dedup mode also rank) gets a 64-bit LDS bitmap of the tile's
// tokens that use it, built with ds_or_b64 (order independent).  popcount of
// the bits below a lane is the token's rank among the tile's earlier users of
// the column; popcount of the whole bitmap is the tile's count.  The tile
// counts are then scanned over tiles, per column, into the absolute first row
// of each tile in each column.  A row's position is base[tile][column] + rank,
// which makes the send buffer order (rank, expert, token) - or (rank, token) -
// stable and deterministic.  No global atomics anywhere.
//
// Two kernels: tile_counts (one wave per tile, so the per-assignment work and
// its memory traffic spread over many CUs) and plan_scan (one workgroup, which
// only reads the per-tile counts, one byte each, and writes the bases).
//
// All global loads are issued unconditionally from clamped, in-bounds
// addresses and only stores are predicated: a load under a branch is followed
// by a wait for it, which would serialise them.
#include "common.hpp"
#include "moe_route.h"

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

// Counts one 64-token tile in the calling wave.  `bits` holds C zeroed
// bitmaps: column c's bit i is set when token i of the tile uses column c.
// Lane l owns the ids at flat positions l + 64 r of the tile (token
// (l + 64 r) / k, slot (l + 64 r) % k) and writes their slot codes back at the
// same positions, so loads and stores stay coalesced.  In dedup mode every id
// also sets its token's bit in its rank's bitmap (setting it twice is harmless).
// `s_rank` maps expert -> rank (LDS) or is null for contiguous placement.
template <bool DEDUP, int KMAX>
__device__ __forceinline__ void count_tile(const int (&raw)[KMAX], int64_t f0, int nf, int k,
                                           uint32_t kmul, int E, const int32_t* s_rank, int m,
                                           uint64_t* bits, uint32_t* __restrict__ lslot,
                                           int lane) {
  int e[KMAX], col[KMAX], tl[KMAX];
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    const int f = lane + kWave * r;
    e[r] = clampi(raw[r], 0, E - 1);
    tl[r] = kdiv(uint32_t(f), kmul, k);
    tl[r] = tl[r] < kTile ? tl[r] : kTile - 1;  // positions past the tile are never used
    col[r] = DEDUP ? (s_rank ? s_rank[e[r]] : e[r] / m) : e[r];
  }
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    if (lane + kWave * r < nf) {
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
    const uint64_t below = tl[r] == 0 ? 0ull : (~0ull >> (kWave - tl[r]));
    code[r] = (uint32_t(col[r]) << 8) | uint32_t(__popcll(mb & below));
  }
#pragma unroll
  for (int r = 0; r < KMAX; ++r)
    if (lane + kWave * r < nf) lslot[f0 + lane + kWave * r] = code[r];
}

// ----------------------------------------------------------- tile counts --

template <bool DEDUP, int KMAX>
__global__ void __launch_bounds__(kWave)
tile_counts_kernel(const int32_t* __restrict__ idx, int64_t T, int E, int k, int R,
                   const int32_t* __restrict__ place, int m, uint32_t kmul,
                   uint8_t* __restrict__ tcnt, uint32_t* __restrict__ lslot) {
  extern __shared__ uint64_t s_tdyn[];
  const int C = E + (DEDUP ? R : 0);
  uint64_t* bits = s_tdyn;                                        // [C]
  int32_t* s_rank = reinterpret_cast<int32_t*>(s_tdyn + C);      // [E] (dedup, explicit placement)
  const int lane = lane_id();
  const int64_t b = blockIdx.x;
  const int64_t f0 = b * kTile * k;
  const int64_t total = T * k;
  const int nf = int(total - f0 < int64_t(kTile) * k ? total - f0 : int64_t(kTile) * k);
  int raw[KMAX];
  load_tile_ids<KMAX>(raw, idx, f0, total, lane);
  for (int c = lane; c < C; c += kWave) bits[c] = 0ull;
  const bool has_rank = DEDUP && place;
  if (has_rank)
    for (int e = lane; e < E; e += kWave) s_rank[e] = clampi(place[e], 0, R - 1);
  wave_lds_sync();
  count_tile<DEDUP, KMAX>(raw, f0, nf, k, kmul, E, has_rank ? s_rank : nullptr, m, bits, lslot,
                          lane);
  for (int c = lane; c < C; c += kWave) tcnt[b * C + c] = uint8_t(__popcll(bits[c]));
}

// ------------------------------------------------------------------- scan --

constexpr int kScanThreads = 1024;
constexpr int kScanWaves = kScanThreads / kWave;
constexpr int kMaxCols = MOE_MAX_EXPERTS + MOE_MAX_RANKS;
constexpr int kScanMaxStaged = 32 * 1024;  // tile-count bytes staged in LDS
constexpr int kMaxQ = 16;                   // tile chunks per column

// Tile counts are read from LDS (STAGED) or straight from global memory.
template <bool STAGED>
__device__ __forceinline__ int tc_at(const uint8_t* __restrict__ g, const uint8_t* s, size_t i) {
  return STAGED ? int(s[i]) : int(g[i]);
}

// Inclusive scan over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(v, off, kWave);
    v += lane >= off ? o : 0;
  }
  return v;
}

// One workgroup: per column, the sum of each chunk of tiles, the chunk's
// prefix and the column total; experts are ordered by (rank, id) with a
// counting sort and one block-wide scan; then every (tile, position column)
// gets its absolute first row.  Loops are short and their loads independent,
// so no phase waits on a chain of LDS round trips.
template <bool DEDUP, bool STAGED>
__global__ void __launch_bounds__(kScanThreads)
plan_scan_kernel(const uint8_t* __restrict__ tcnt, int B, int E, int R,
                 const int32_t* __restrict__ place, int m, int32_t* __restrict__ expert_counts,
                 int32_t* __restrict__ rank_counts, int32_t* __restrict__ rank_offsets,
                 int32_t* __restrict__ expert_offsets, int32_t* __restrict__ header,
                 int32_t* __restrict__ base) {
  extern __shared__ u32x4 s_tc4[];
  __shared__ int32_t s_part[kMaxCols];       // [q][c] chunk sums
  __shared__ int32_t s_pre[kMaxCols];        // [q][c] chunk prefixes
  __shared__ int32_t s_tot[kMaxCols];        // column totals
  __shared__ int32_t s_colbase[MOE_MAX_EXPERTS];
  __shared__ int32_t s_sorted[MOE_MAX_EXPERTS];
  __shared__ uint64_t s_rmask[MOE_MAX_RANKS][MOE_MAX_EXPERTS / kWave];
  __shared__ int32_t s_rcnt[MOE_MAX_RANKS];
  __shared__ int32_t s_rstart[MOE_MAX_RANKS + 1];
  __shared__ int32_t s_ro[MOE_MAX_RANKS + 1];
  __shared__ int32_t s_wsum[kScanWaves];
  const uint8_t* s_tc = reinterpret_cast<const uint8_t*>(s_tc4);
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid / kWave;
  const int C = E + (DEDUP ? R : 0);
  const int CP = DEDUP ? R : E;
  const int cbase = DEDUP ? E : 0;  // first position column among the counted ones
  int Q = kScanThreads / C;
  Q = Q < 1 ? 1 : (Q > kMaxQ ? kMaxQ : Q);
  const int units = C * Q;
  const int EW = (E + kWave - 1) / kWave;  // 64-expert words
  const bool sorted_by_id = DEDUP || place == nullptr;  // (rank, id) order == id order

  // 0. stage the tile counts (16-byte vectors, all loads before any LDS store)
  if (STAGED) {
    const int nvec = (B * C + 15) / 16;
    const u32x4* g4 = reinterpret_cast<const u32x4*>(tcnt);
    for (int v0 = 0; v0 < nvec; v0 += 4 * kScanThreads) {
      u32x4 tmp[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int v = v0 + u * kScanThreads + tid;
        tmp[u] = g4[v < nvec ? v : nvec - 1];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int v = v0 + u * kScanThreads + tid;
        if (v < nvec) s_tc4[v] = tmp[u];
      }
    }
  }
  // rank of the experts this thread owns (place is wave-uniform: scalar branch)
  int my_rank = 0;
  if (tid < E) my_rank = place ? clampi(place[tid], 0, R - 1) : tid / m;
  if (tid < MOE_MAX_RANKS) s_rcnt[tid] = 0;
  for (int i = tid; i < MOE_MAX_RANKS * (MOE_MAX_EXPERTS / kWave); i += kScanThreads)
    (&s_rmask[0][0])[i] = 0ull;
  __syncthreads();

  // 1. chunk sums per (column, chunk); rank membership of each expert
  for (int u = tid; u < units; u += kScanThreads) {
    const int c = u % C, q = u / C;
    const int b0 = int(int64_t(B) * q / Q), b1 = int(int64_t(B) * (q + 1) / Q);
    int32_t sum = 0;
#pragma unroll 8
    for (int b = b0; b < b1; ++b) sum += tc_at<STAGED>(tcnt, s_tc, size_t(b) * C + c);
    s_part[u] = sum;
  }
  if (!sorted_by_id && tid < E) {
    atomicOr(reinterpret_cast<unsigned long long*>(&s_rmask[my_rank][tid / kWave]),
             1ull << (tid % kWave));
    atomicAdd(&s_rcnt[my_rank], 1);
  }
  __syncthreads();

  // 2. chunk prefixes and column totals; start of each rank in the expert order
  for (int u = tid; u < units; u += kScanThreads) {
    const int c = u % C, q = u / C;
    int32_t pre = 0;
#pragma unroll
    for (int qq = 0; qq < kMaxQ; ++qq) pre += qq < q ? s_part[(qq < Q ? qq : 0) * C + c] : 0;
    s_pre[u] = pre;
    if (q == Q - 1) s_tot[c] = pre + s_part[u];
  }
  if (!sorted_by_id && w == 0) {
    const int v = lane < R ? s_rcnt[lane] : 0;
    const int incl = wave_incl_scan(v);
    if (lane < R) s_rstart[lane] = incl - v;
  }
  __syncthreads();

  // 3. the expert order: expert e goes to slot `key` of the (rank, id) order
  int key = tid;
  if (!sorted_by_id && tid < E) {
    const uint64_t* mk = s_rmask[my_rank];
    const int wi = tid / kWave;
    int below = __popcll(mk[wi] & lanemask_lt());
#pragma unroll
    for (int q = 0; q < MOE_MAX_EXPERTS / kWave; ++q) below += q < wi ? __popcll(mk[q]) : 0;
    key = s_rstart[my_rank] + below;
  }
  if (!DEDUP && tid < E) s_sorted[key] = s_tot[tid];
  __syncthreads();

  // 4. exclusive scan in that order (experts, or ranks in dedup mode)
  const int nscan = DEDUP ? R : E;
  int v = 0;
  if (tid < nscan) v = DEDUP ? s_tot[E + tid] : s_sorted[tid];
  int incl = 0;
  if (w < (nscan + kWave - 1) / kWave) {
    incl = wave_incl_scan(v);
    if (lane == kWave - 1) s_wsum[w] = incl;
  }
  __syncthreads();
  int carry = 0;
#pragma unroll
  for (int q = 0; q < kScanWaves; ++q) carry += q < w ? s_wsum[q < EW ? q : 0] : 0;
  const int excl = carry + incl - v;
  if (tid < nscan) s_sorted[tid] = excl;  // scanned value of slot tid
  if (tid == 0) {
    int total = 0;
#pragma unroll
    for (int q = 0; q < kScanWaves; ++q) total += q < (nscan + kWave - 1) / kWave ? s_wsum[q] : 0;
    s_ro[R] = total;
    header[0] = total;
  }
  __syncthreads();

  // 5. counts, offsets and column bases
  if (tid < E) expert_counts[tid] = s_tot[tid];
  if (!DEDUP) {
    if (tid < E) {
      const int off = s_sorted[key];
      s_colbase[tid] = off;
      if (expert_offsets) expert_offsets[tid] = off;
    }
    if (tid < R) {
      // the first expert of rank r in the (rank, id) order
      const int first = sorted_by_id ? tid * m : s_rstart[tid];
      s_ro[tid] = first < E ? s_sorted[first] : s_ro[R];
    }
  } else if (tid < R) {
    s_ro[tid] = s_sorted[tid];
    s_colbase[tid] = s_sorted[tid];
  }
  __syncthreads();
  if (tid < R) rank_counts[tid] = s_ro[tid + 1] - s_ro[tid];
  if (tid <= R) rank_offsets[tid] = s_ro[tid];

  // 6. absolute first row of every (tile, position column)
  for (int u = tid; u < CP * Q; u += kScanThreads) {
    const int cp = u % CP, q = u / CP;
    const int c = cbase + cp;
    const int b0 = int(int64_t(B) * q / Q), b1 = int(int64_t(B) * (q + 1) / Q);
    int32_t run = s_colbase[cp] + s_pre[q * C + c];
    for (int b = b0; b < b1; ++b) {
      base[size_t(b) * CP + cp] = run;
      run += tc_at<STAGED>(tcnt, s_tc, size_t(b) * C + c);
    }
  }
}

template <int KMAX>
static hipError_t launch_counts_k(const int32_t* idx, int64_t T, int E, int k, int R,
                                  const int32_t* place, int dedup, int32_t* expert_counts,
                                  int32_t* rank_counts, int32_t* rank_offsets,
                                  int32_t* expert_offsets, void* workspace, hipStream_t stream) {
  const PlanLayout pl = plan_layout(T, E, k, R, dedup);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* header = reinterpret_cast<int32_t*>(ws);
  int32_t* base = reinterpret_cast<int32_t*>(ws + pl.base_off);
  uint8_t* tcnt = ws + pl.tcnt_off;
  uint32_t* lslot = reinterpret_cast<uint32_t*>(ws + pl.lslot_off);
  const int m = E / R;
  if (T > 0) {
    const size_t lds = size_t(pl.cols) * sizeof(uint64_t) + size_t(E) * sizeof(int32_t);
    const uint32_t kmul = kdiv_mul(k);
    if (dedup)
      hipLaunchKernelGGL((tile_counts_kernel<true, KMAX>), dim3(unsigned(pl.tiles)), dim3(kWave),
                         lds, stream, idx, T, E, k, R, place, m, kmul, tcnt, lslot);
    else
      hipLaunchKernelGGL((tile_counts_kernel<false, KMAX>), dim3(unsigned(pl.tiles)),
                         dim3(kWave), lds, stream, idx, T, E, k, R, place, m, kmul, tcnt, lslot);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int B = int(pl.tiles);
  const size_t staged = size_t(B) * pl.cols;
  const bool fits = staged <= size_t(kScanMaxStaged);
  const size_t lds = fits ? ((staged + 15) / 16) * 16 : 0;
#define MOE_SCAN_LAUNCH(D, S)                                                                   \
  hipLaunchKernelGGL((plan_scan_kernel<D, S>), dim3(1), dim3(kScanThreads), lds, stream, tcnt, B, \
                     E, R, place, m, expert_counts, rank_counts, rank_offsets, expert_offsets,    \
                     header, base)
  if (dedup) {
    if (fits) MOE_SCAN_LAUNCH(true, true);
    else MOE_SCAN_LAUNCH(true, false);
  } else {
    if (fits) MOE_SCAN_LAUNCH(false, true);
    else MOE_SCAN_LAUNCH(false, false);
  }
#undef MOE_SCAN_LAUNCH
  return hipGetLastError();
}

hipError_t launch_send_counts(const int32_t* idx, int64_t T, int E, int k, int R,
                              const int32_t* place, int dedup, int32_t* expert_counts,
                              int32_t* rank_counts, int32_t* rank_offsets,
                              int32_t* expert_offsets, void* workspace, hipStream_t stream) {
  if (k <= 2)
    return launch_counts_k<2>(idx, T, E, k, R, place, dedup, expert_counts, rank_counts,
                              rank_offsets, expert_offsets, workspace, stream);
  if (k <= 4)
    return launch_counts_k<4>(idx, T, E, k, R, place, dedup, expert_counts, rank_counts,
                              rank_offsets, expert_offsets, workspace, stream);
  if (k <= 8)
    return launch_counts_k<8>(idx, T, E, k, R, place, dedup, expert_counts, rank_counts,
                              rank_offsets, expert_offsets, workspace, stream);
  return launch_counts_k<16>(idx, T, E, k, R, place, dedup, expert_counts, rank_counts,
                             rank_offsets, expert_offsets, workspace, stream);
}

}  // namespace moe
