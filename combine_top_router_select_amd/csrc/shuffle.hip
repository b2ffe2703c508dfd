// Token-shuffle planner: fit and prediction (GPU).  The capacity-constrained
// assignment that follows is host code, in placement.hip.
//
// Source: "Expert Coupling in MoE Pretraining" (summary), "Method 2: Token
// Shuffling": the planner predicts each token's owner rank at layer l+1 from
// the experts it selected at the two preceding MoE layers - a pair lookup
// with a single-expert fallback for sparse observations - and, since every
// rank must own exactly T/EP tokens, assigns tokens in decreasing confidence
// to their most preferred rank with room left.  The page prints no formula;
// the readings (tables of rank counts, score = sum of the pairs' rank
// distributions, confidence = largest score / sum of scores) are stated in
// include/moe_route.h.
//
// fit: one lane per token; every (a, b) pair of its layer l-1 and layer l
// experts adds, for every rank r, the number of its layer l+1 experts placed
// on r (integer atomics: exact in any order).
// predict: one wave per token, lane r = rank r (R <= 64).  The k x k pair
// rows and fallback rows are loaded in batches before any arithmetic; each
// row's total is a wave-wide integer sum; the scores are summed in fp64 in
// (slot of a, slot of b) order and rounded once, so they equal the oracle's
// bit for bit and the assignment's decisions are the same.
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

constexpr int kPredBatch = 8;  // pairs whose rows are loaded together

__device__ __forceinline__ int wave_sum_int(int v) {
  return __builtin_amdgcn_readlane(wave_incl_scan(v), kWave - 1);
}

__global__ void __launch_bounds__(256)
shuffle_predict_kernel(const int32_t* __restrict__ prev, const int32_t* __restrict__ cur,
                       int64_t T, int E, int k, int R, const int32_t* __restrict__ pair,
                       const int32_t* __restrict__ single, int min_obs,
                       float* __restrict__ scores) {
  const int lane = lane_id();
  const int64_t t = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;
  if (t >= T) return;  // whole wave
  const int r = lane < R ? lane : R - 1;
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
      const int p = lane < R ? pv[i] : 0, s = lane < R ? sv[i] : 0;
      const int n = wave_sum_int(p);
      if (n >= min_obs && n > 0) {
        sc += double(p) / double(n);
      } else {
        const int msum = wave_sum_int(s);
        if (msum > 0) sc += double(s) / double(msum);
      }
    }
  }
  if (lane < R) scores[t * R + lane] = float(sc);
}

hipError_t launch_shuffle_fit(const int32_t* prev, const int32_t* cur, const int32_t* next,
                              int64_t T, int E, int k, int R, const int32_t* place,
                              int32_t* pair, int32_t* single, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(shuffle_fit_kernel, dim3(unsigned((T + 255) / 256)), dim3(256), 0, stream,
                     prev, cur, next, T, E, k, R, place, E / R, pair, single);
  return hipGetLastError();
}

hipError_t launch_shuffle_predict(const int32_t* prev, const int32_t* cur, int64_t T, int E,
                                  int k, int R, const int32_t* pair, const int32_t* single,
                                  int min_obs, float* scores, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(shuffle_predict_kernel, dim3(unsigned((T + 3) / 4)), dim3(256), 0, stream,
                     prev, cur, T, E, k, R, pair, single, min_obs, scores);
  return hipGetLastError();
}

}  // namespace moe
