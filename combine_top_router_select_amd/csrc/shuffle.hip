// Token-shuffle planner: fit and prediction (GPU).  The capacity-constrained
// assignment that follows is host code, in placement.hip.
//
// Source: "Expert Coupling in MoE Pretraining" (summary), "Method 2: Token
// Shuffling".  Reading: the rank that will serve a token at the next MoE layer
// is guessed from the two expert choices it made at the two layers before
// (the pair of choices, or the later choice alone when that pair has been seen
// too few times); ranks then take equal shares of the tokens, the surest
// guesses placed first.  No formula is printed; the readings (tables of rank
// counts, score = sum of the pairs' rank distributions, confidence = largest
// score / sum of scores) are stated in include/moe_route.h.
//
// fit: the tables in LDS when a row of E x R counts fits (each workgroup owns
// a range of layer l-1 experts, scans all tokens and adds its rows to the
// global table once); else one lane per token with global atomics.  Integer
// sums: exact in any order.
// predict: R lanes per token (rounded up to a power of two), lane r = rank r.
// The k x k pair rows and fallback rows are loaded in batches before any
// arithmetic; each row's total is an integer sum over the token's lanes; the
// scores are summed in fp64 in (slot of a, slot of b) order and rounded once,
// so they equal the oracle's bit for bit and the assignment's decisions are
// the same.
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"
#include "moe_route.h"

namespace moe {

__global__ void __launch_bounds__(256)
shuffle_fit_kernel(const int32_t* __restrict__ prev, const int32_t* __restrict__ cur,
                   const int32_t* __restrict__ next, int64_t T, int E, int k, int R,
                   const int32_t* __restrict__ place, int m, int32_t* __restrict__ pair,
                   int32_t* __restrict__ single) {
  const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= T) return;
  int rk[MOE_MAX_TOP_K], rc[MOE_MAX_TOP_K];  // distinct ranks of the layer l+1 experts
  int nr = 0;
  for (int j = 0; j < k; ++j) {
    const int c = clampi(next[t * k + j], 0, E - 1);
    const int r = place ? clampi(place[c], 0, R - 1) : c / m;
    int i = 0;
    while (i < nr && rk[i] != r) ++i;
    if (i == nr) {
      rk[nr] = r;
      rc[nr] = 0;
      ++nr;
    }
    ++rc[i];
  }
  for (int jb = 0; jb < k; ++jb) {
    const int b = clampi(cur[t * k + jb], 0, E - 1);
    for (int i = 0; i < nr; ++i) atomicAdd(&single[int64_t(b) * R + rk[i]], rc[i]);
    for (int ja = 0; ja < k; ++ja) {
      const int a = clampi(prev[t * k + ja], 0, E - 1);
      int32_t* row = pair + (int64_t(a) * E + b) * R;
      for (int i = 0; i < nr; ++i) atomicAdd(&row[rk[i]], rc[i]);
    }
  }
}

// The fit with the tables in LDS, for a grid of (layer l-1 expert range g,
// token slice s): workgroup (g, s) counts, in LDS, the pair-table rows
// a in [g A, g A + A) (A rows of E x R counts fill at most kFitPairLds bytes)
// from the kFitTok tokens of slice s - a token adds one LDS atomic per
// (a, b, slot of c) for its layer l-1 experts in the range (a repeated rank
// just adds 1 more than once) - and, when g == s % G, the slice's
// single-expert counts (kFitPerThread tokens per thread).  The non-zero LDS
// counts are then added to the global tables: with plain read-modify-writes
// for the pair rows when there is one slice (no other workgroup touches them),
// else with global atomics.  Used when an E x R row fits kFitSingleLds; else
// the one-lane-per-token kernel above.
constexpr int kFitThreads = 256;
constexpr int kFitPerThread = 4;
constexpr int kFitTok = kFitThreads * kFitPerThread;  // tokens per slice
constexpr size_t kFitPairLds = 48 * 1024;
constexpr size_t kFitSingleLds = 16 * 1024;

__global__ void __launch_bounds__(kFitThreads)
shuffle_fit_lds_kernel(const int32_t* __restrict__ prev, const int32_t* __restrict__ cur,
                       const int32_t* __restrict__ next, int64_t T, int E, int k, int R,
                       const int32_t* __restrict__ place, int m, int A,
                       int32_t* __restrict__ pair, int32_t* __restrict__ single) {
  extern __shared__ int32_t s_fit[];
  const int ER = E * R;
  int32_t* s_pair = s_fit;             // [A][E][R]
  int32_t* s_single = s_fit + A * ER;  // [E][R]
  const int tid = threadIdx.x;
  const int G = int(gridDim.x), g = int(blockIdx.x);
  const int64_t sl = blockIdx.y;
  const bool own_single = g == int(sl % G);
  const int a0 = g * A;
  const int na = E - a0 < A ? E - a0 : A;
  for (int q = tid; q < (A + 1) * ER; q += kFitThreads) s_fit[q] = 0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kFitPerThread; ++u) {
    const int64_t t = sl * kFitTok + u * kFitThreads + tid;
    if (t >= T) break;
    uint32_t amask = 0;  // slots of the token's layer l-1 experts in this workgroup's rows
    for (int ja = 0; ja < k; ++ja) {
      const int a = clampi(prev[t * k + ja], 0, E - 1);
      amask |= (a >= a0 && a < a0 + na) ? (1u << ja) : 0u;
    }
    if (amask == 0 && !own_single) continue;
    int rr[MOE_MAX_TOP_K];  // rank of each layer l+1 expert
#pragma unroll
    for (int jc = 0; jc < MOE_MAX_TOP_K; ++jc) {
      if (jc < k) {
        const int c = clampi(next[t * k + jc], 0, E - 1);
        rr[jc] = place ? clampi(place[c], 0, R - 1) : c / m;
      }
    }
    for (int jb = 0; jb < k; ++jb) {
      const int b = clampi(cur[t * k + jb], 0, E - 1);
      if (own_single) {
#pragma unroll
        for (int jc = 0; jc < MOE_MAX_TOP_K; ++jc)
          if (jc < k) atomicAdd(&s_single[b * R + rr[jc]], 1);
      }
      for (uint32_t am = amask; am; am &= am - 1) {
        const int a = clampi(prev[t * k + (__ffs(am) - 1)], 0, E - 1);
        int32_t* row = s_pair + ((a - a0) * E + b) * R;
#pragma unroll
        for (int jc = 0; jc < MOE_MAX_TOP_K; ++jc)
          if (jc < k) atomicAdd(&row[rr[jc]], 1);
      }
    }
  }
  __syncthreads();
  int32_t* grow = pair + int64_t(a0) * ER;
  const bool sole = gridDim.y == 1;
  for (int q = tid; q < na * ER; q += kFitThreads) {
    const int v = s_pair[q];
    if (v) {
      if (sole) grow[q] += v;  // the only writer of these rows
      else atomicAdd(&grow[q], v);
    }
  }
  if (own_single)
    for (int q = tid; q < ER; q += kFitThreads) {
      const int v = s_single[q];
      if (v) atomicAdd(&single[q], v);
    }
}

constexpr int kPredBatch = 8;  // pairs whose rows are loaded together

// Sum over aligned segments of S lanes (S a power of two <= 64); every lane of
// a segment gets it.  Integer, so exact in any order.
template <int S>
__device__ __forceinline__ int segment_sum(int v) {
  if (S >= 2) v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm xor 1
  if (S >= 4) v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm xor 2
  if (S >= 8) v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  if (S >= 16) v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false); // row_mirror
  if (S >= 32) v += __shfl_xor(v, 16, kWave);
  if (S >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

// S lanes per token (S = R rounded up to a power of two), lane r of a segment =
// rank r, so a wave scores 64 / S tokens.  Per pair the row totals are segment
// sums taken by every lane (no cross-lane operation under a lane-divergent
// branch), and each rank's score is summed in fp64 in the oracle's order.
template <int S>
__global__ void __launch_bounds__(256)
shuffle_predict_kernel(const int32_t* __restrict__ prev, const int32_t* __restrict__ cur,
                       int64_t T, int E, int k, int R, const int32_t* __restrict__ pair,
                       const int32_t* __restrict__ single, int min_obs,
                       float* __restrict__ scores) {
  const int lane = lane_id();
  const int64_t wave = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;
  const int64_t t_raw = wave * (kWave / S) + lane / S;
  if (wave * (kWave / S) >= T) return;  // whole wave
  const bool tok_ok = t_raw < T;
  const int64_t t = tok_ok ? t_raw : T - 1;  // loads stay in bounds
  const int rl = lane & (S - 1);
  const bool rank_ok = tok_ok && rl < R;
  const int r = rl < R ? rl : R - 1;
  const int kk = k * k;
  double sc = 0.0;
  for (int q0 = 0; q0 < kk; q0 += kPredBatch) {
    int pv[kPredBatch], sv[kPredBatch];
#pragma unroll
    for (int i = 0; i < kPredBatch; ++i) {
      const int q = q0 + i < kk ? q0 + i : kk - 1;
      const int a = clampi(prev[t * k + q / k], 0, E - 1);
      const int b = clampi(cur[t * k + q % k], 0, E - 1);
      pv[i] = pair[(int64_t(a) * E + b) * R + r];
      sv[i] = single[int64_t(b) * R + r];
    }
#pragma unroll
    for (int i = 0; i < kPredBatch; ++i) {
      if (q0 + i >= kk) break;  // wave-uniform
      const int p = rank_ok ? pv[i] : 0, s1 = rank_ok ? sv[i] : 0;
      const int n = segment_sum<S>(p);
      const int ms = segment_sum<S>(s1);
      const bool use_pair = n >= min_obs && n > 0;
      const int num = use_pair ? p : s1;
      const int den = use_pair ? n : ms;
      if (den > 0) sc += double(num) / double(den);
    }
  }
  if (rank_ok) scores[t * R + rl] = float(sc);
}

hipError_t launch_shuffle_fit(const int32_t* prev, const int32_t* cur, const int32_t* next,
                              int64_t T, int E, int k, int R, const int32_t* place,
                              int32_t* pair, int32_t* single, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const size_t row_bytes = size_t(E) * size_t(R) * sizeof(int32_t);  // one a: E x R counts
  if (row_bytes <= kFitSingleLds) {
    const int A = int(kFitPairLds / row_bytes);
    const int G = (E + A - 1) / A;
    const int64_t S = (T + kFitTok - 1) / kFitTok;
    if (S <= 65535) {
      hipLaunchKernelGGL(shuffle_fit_lds_kernel, dim3(unsigned(G), unsigned(S)),
                         dim3(kFitThreads), (size_t(A) + 1) * row_bytes, stream, prev, cur, next,
                         T, E, k, R, place, E / R, A, pair, single);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL(shuffle_fit_kernel, dim3(unsigned((T + 255) / 256)), dim3(256), 0, stream,
                     prev, cur, next, T, E, k, R, place, E / R, pair, single);
  return hipGetLastError();
}

hipError_t launch_shuffle_predict(const int32_t* prev, const int32_t* cur, int64_t T, int E,
                                  int k, int R, const int32_t* pair, const int32_t* single,
                                  int min_obs, float* scores, hipStream_t stream) {
  if (T == 0) return hipSuccess;
#define MOE_PRED(SS)                                                                      \
  do {                                                                                    \
    const int64_t waves = (T + (kWave / SS) - 1) / (kWave / SS);                          \
    hipLaunchKernelGGL(shuffle_predict_kernel<SS>, dim3(unsigned((waves + 3) / 4)),       \
                       dim3(256), 0, stream, prev, cur, T, E, k, R, pair, single,         \
                       min_obs, scores);                                                  \
  } while (0)
  if (R <= 1) MOE_PRED(1);
  else if (R <= 2) MOE_PRED(2);
  else if (R <= 4) MOE_PRED(4);
  else if (R <= 8) MOE_PRED(8);
  else if (R <= 16) MOE_PRED(16);
  else if (R <= 32) MOE_PRED(32);
  else MOE_PRED(64);
#undef MOE_PRED
  return hipGetLastError();
}

}  // namespace moe
