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
// Two kernels, no global atomics:
//  1. tile_counts: one wave per 64-token tile, one lane per token.  Each column
//     (expert; in dedup mode also rank) gets a 64-bit LDS bitmap of the tile's
//     tokens that use it (ds_or_b64 - order independent).  popcount of the bits
//     below a lane is the token's rank among the tile's earlier users of that
//     column; popcount of the whole bitmap is the tile's count.
//  2. plan_scan: one 1024-thread workgroup scans the tile counts of every
//     column (chunked over tiles), derives expert/rank counts and offsets, and
//     rewrites each tile count into the absolute first row of that tile in that
//     column.  A row's position is then base[tile][column] + lrank, which makes
//     the send buffer order (rank, expert, token) - or (rank, token) - stable
//     and deterministic.
#include "common.hpp"

namespace moe {

__device__ __forceinline__ int rank_of(int e, const int32_t* place, int m, int R) {
  return place ? clampi(place[e], 0, R - 1) : e / m;
}

template <bool DEDUP>
__global__ void __launch_bounds__(256)
tile_counts_kernel(const int32_t* __restrict__ idx, int64_t T, int E, int k, int R,
                   const int32_t* __restrict__ place, int m, int32_t* __restrict__ base,
                   uint8_t* __restrict__ lrank, int64_t B) {
  extern __shared__ uint64_t s_bits[];
  const int C = E + (DEDUP ? R : 0);
  const int w = threadIdx.x / kWave;
  const int lane = lane_id();
  uint64_t* sel = s_bits + size_t(w) * C;
  const int64_t b = int64_t(blockIdx.x) * (blockDim.x / kWave) + w;
  for (int c = lane; c < C; c += kWave) sel[c] = 0ull;
  __syncthreads();
  const bool active = b < B;
  const int64_t t = b * kTile + lane;
  const bool valid = active && t < T;
  const uint64_t bit = 1ull << lane;
  if (valid) {
    uint64_t rmask = 0ull;
    for (int j = 0; j < k; ++j) {
      const int e = clampi(idx[t * k + j], 0, E - 1);
      atomicOr(reinterpret_cast<unsigned long long*>(&sel[e]), (unsigned long long)bit);
      if (DEDUP) rmask |= 1ull << rank_of(e, place, m, R);
    }
    if (DEDUP) {
      while (rmask) {
        const int r = __ffsll((unsigned long long)rmask) - 1;
        rmask &= rmask - 1;
        atomicOr(reinterpret_cast<unsigned long long*>(&sel[E + r]), (unsigned long long)bit);
      }
    }
  }
  __syncthreads();
  const uint64_t lt = lanemask_lt();
  if (valid) {
    for (int j = 0; j < k; ++j) {
      const int e = clampi(idx[t * k + j], 0, E - 1);
      const int col = DEDUP ? E + rank_of(e, place, m, R) : e;
      lrank[t * k + j] = uint8_t(__popcll(sel[col] & lt));
    }
  }
  if (active)
    for (int c = lane; c < C; c += kWave) base[b * C + c] = __popcll(sel[c]);
}

constexpr int kScanThreads = 1024;
constexpr int kMaxCols = 1024 + 64;

template <bool DEDUP>
__global__ void __launch_bounds__(kScanThreads)
plan_scan_kernel(int32_t* __restrict__ base, int64_t B, int E, int R,
                 const int32_t* __restrict__ place, int m, int32_t* __restrict__ expert_counts,
                 int32_t* __restrict__ rank_counts, int32_t* __restrict__ rank_offsets,
                 int32_t* __restrict__ expert_offsets, int32_t* __restrict__ header) {
  __shared__ int32_t s_part[kMaxCols];   // chunk prefixes, [q][c]
  __shared__ int32_t s_tot[kMaxCols];    // column totals
  __shared__ int32_t s_colbase[kMaxCols];
  __shared__ int32_t s_place[1024];
  __shared__ int32_t s_rc[64];
  __shared__ int32_t s_ro[65];
  const int tid = threadIdx.x;
  const int C = E + (DEDUP ? R : 0);
  const int Q = C >= kScanThreads ? 1 : kScanThreads / C;  // tile chunks per column
  const int units = C * Q;

  for (int e = tid; e < E; e += kScanThreads) s_place[e] = rank_of(e, place, m, R);
  if (tid < 64) s_rc[tid] = 0;
  // 1. per (column, chunk) sums of the tile counts
  for (int u = tid; u < units; u += kScanThreads) {
    const int c = u % C, q = u / C;
    const int64_t b0 = B * q / Q, b1 = B * (q + 1) / Q;
    int32_t s = 0;
    for (int64_t b = b0; b < b1; ++b) s += base[b * C + c];
    s_part[u] = s;
  }
  __syncthreads();
  // 2. exclusive prefix over chunks, column totals
  for (int c = tid; c < C; c += kScanThreads) {
    int32_t run = 0;
    for (int q = 0; q < Q; ++q) {
      const int32_t v = s_part[q * C + c];
      s_part[q * C + c] = run;
      run += v;
    }
    s_tot[c] = run;
  }
  __syncthreads();
  // 3. counts and offsets
  for (int e = tid; e < E; e += kScanThreads) {
    expert_counts[e] = s_tot[e];
    if (!DEDUP) atomicAdd(&s_rc[s_place[e]], s_tot[e]);  // integer: order independent
  }
  if (DEDUP && tid < R) s_rc[tid] = s_tot[E + tid];
  __syncthreads();
  if (tid == 0) {
    int32_t run = 0;
    for (int r = 0; r < R; ++r) {
      s_ro[r] = run;
      run += s_rc[r];
    }
    s_ro[R] = run;
    header[0] = run;
  }
  __syncthreads();
  if (tid < R) rank_counts[tid] = s_rc[tid];
  if (tid <= R) rank_offsets[tid] = s_ro[tid];
  if (!DEDUP) {
    // experts inside a rank in ascending id
    for (int e = tid; e < E; e += kScanThreads) {
      const int r = s_place[e];
      int32_t off = s_ro[r];
      for (int e2 = 0; e2 < e; ++e2)
        if (s_place[e2] == r) off += s_tot[e2];
      s_colbase[e] = off;
      if (expert_offsets) expert_offsets[e] = off;
    }
  } else {
    for (int r = tid; r < R; r += kScanThreads) s_colbase[E + r] = s_ro[r];
  }
  __syncthreads();
  // 4. absolute first row of every (tile, column) that dispatch uses
  for (int u = tid; u < units; u += kScanThreads) {
    const int c = u % C, q = u / C;
    if (DEDUP && c < E) continue;
    const int64_t b0 = B * q / Q, b1 = B * (q + 1) / Q;
    int32_t run = s_colbase[c] + s_part[u];
    for (int64_t b = b0; b < b1; ++b) {
      const int32_t v = base[b * C + c];
      base[b * C + c] = run;
      run += v;
    }
  }
}

hipError_t launch_send_counts(const int32_t* idx, int64_t T, int E, int k, int R,
                              const int32_t* place, int dedup, int32_t* expert_counts,
                              int32_t* rank_counts, int32_t* rank_offsets,
                              int32_t* expert_offsets, void* workspace, hipStream_t stream) {
  const PlanLayout pl = plan_layout(T, E, k, R, dedup);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* header = reinterpret_cast<int32_t*>(ws);
  int32_t* base = reinterpret_cast<int32_t*>(ws + pl.base_off);
  uint8_t* lrank = ws + pl.lrank_off;
  const int m = E / R;
  if (T > 0) {
    const int64_t blocks = (pl.tiles + 3) / 4;
    const size_t lds = size_t(4) * pl.cols * sizeof(uint64_t);
    if (dedup)
      hipLaunchKernelGGL((tile_counts_kernel<true>), dim3(unsigned(blocks)), dim3(256), lds, stream,
                         idx, T, E, k, R, place, m, base, lrank, pl.tiles);
    else
      hipLaunchKernelGGL((tile_counts_kernel<false>), dim3(unsigned(blocks)), dim3(256), lds,
                         stream, idx, T, E, k, R, place, m, base, lrank, pl.tiles);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (dedup)
    hipLaunchKernelGGL((plan_scan_kernel<true>), dim3(1), dim3(kScanThreads), 0, stream, base,
                       pl.tiles, E, R, place, m, expert_counts, rank_counts, rank_offsets,
                       expert_offsets, header);
  else
    hipLaunchKernelGGL((plan_scan_kernel<false>), dim3(1), dim3(kScanThreads), 0, stream, base,
                       pl.tiles, E, R, place, m, expert_counts, rank_counts, rank_offsets,
                       expert_offsets, header);
  return hipGetLastError();
}

}  // namespace moe
