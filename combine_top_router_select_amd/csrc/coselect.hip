// A6 - expert co-selection counts W[E][E].
//
// Source: "Expert Coupling in MoE Pretraining" (summary), "Method 1": the
// correlation graph W[e][e'] counts the tokens that select both e and e'; it is
// the input of the placement search.  "Correlation Formation and Stability":
// about 4096 tokens (one micro-batch of one rank) suffice to fit it.
// The diagonal W[e][e] counts the tokens selecting e (a reading; it does not
// change any placement objective).
//
// Design: W is symmetric, so a workgroup counts only the upper triangle
// (a <= b) in an LDS histogram (integer atomics, order independent, 64 KiB at
// E = 128), then adds it to both halves of W in global memory.  One workgroup
// handles up to kCoselTokens tokens; with a single workgroup the flush is a
// plain read-add-write (one writer per cell), otherwise integer atomics.
// E > 128 does not fit the LDS histogram and counts straight into global memory
// with integer atomics.
#include "common.hpp"

namespace moe {

constexpr int kCoselThreads = 1024;
constexpr int kCoselTokens = 8192;
constexpr int kCoselLdsExperts = 128;

__global__ void __launch_bounds__(kCoselThreads)
coselect_lds_kernel(const int32_t* __restrict__ idx, int64_t n, int E, int k,
                    int32_t* __restrict__ W, int single) {
  extern __shared__ int32_t s_h[];
  const int tid = threadIdx.x;
  for (int i = tid; i < E * E; i += kCoselThreads) s_h[i] = 0;
  __syncthreads();
  const int64_t t_begin = int64_t(blockIdx.x) * kCoselTokens;
  int64_t t_end = t_begin + kCoselTokens;
  if (t_end > n) t_end = n;
  for (int64_t t = t_begin + tid; t < t_end; t += kCoselThreads) {
    const int32_t* ti = idx + t * k;
    for (int a = 0; a < k; ++a) {
      const int ea = clampi(ti[a], 0, E - 1);
      atomicAdd(&s_h[ea * E + ea], 1);
      for (int b = a + 1; b < k; ++b) {
        const int eb = clampi(ti[b], 0, E - 1);
        const int lo = ea < eb ? ea : eb, hi = ea < eb ? eb : ea;
        atomicAdd(&s_h[lo * E + hi], 1);
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < E * E; i += kCoselThreads) {
    const int a = i / E, b = i - a * E;
    if (a > b) continue;
    const int32_t v = s_h[i];
    if (v == 0) continue;
    if (single) {
      W[a * E + b] += v;
      if (a != b) W[b * E + a] += v;
    } else {
      atomicAdd(&W[a * E + b], v);
      if (a != b) atomicAdd(&W[b * E + a], v);
    }
  }
}

__global__ void __launch_bounds__(256)
coselect_global_kernel(const int32_t* __restrict__ idx, int64_t n, int E, int k,
                       int32_t* __restrict__ W) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; t < n; t += stride) {
    const int32_t* ti = idx + t * k;
    for (int a = 0; a < k; ++a) {
      const int ea = clampi(ti[a], 0, E - 1);
      atomicAdd(&W[int64_t(ea) * E + ea], 1);
      for (int b = a + 1; b < k; ++b) {
        const int eb = clampi(ti[b], 0, E - 1);
        atomicAdd(&W[int64_t(ea) * E + eb], 1);
        atomicAdd(&W[int64_t(eb) * E + ea], 1);
      }
    }
  }
}

hipError_t launch_coselect(const int32_t* idx, int64_t n, int E, int k, int32_t* W,
                           hipStream_t stream) {
  if (n == 0) return hipSuccess;
  if (E <= kCoselLdsExperts) {
    const int64_t blocks = (n + kCoselTokens - 1) / kCoselTokens;
    const size_t lds = size_t(E) * E * sizeof(int32_t);
    hipLaunchKernelGGL(coselect_lds_kernel, dim3(unsigned(blocks)), dim3(kCoselThreads), lds,
                       stream, idx, n, E, k, W, blocks == 1 ? 1 : 0);
  } else {
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(coselect_global_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, idx,
                       n, E, k, W);
  }
  return hipGetLastError();
}

}  // namespace moe
