// A1 - top-k routing with softmax gates over the selected logits.
//
// Source: "Expert Coupling in MoE Pretraining" (summary page), section
// "Background": every token goes to its k highest-scoring experts.  The gate is
// the softmax over the k selected logits (the pages speak of routing
// probabilities without a formula; this is the plainest reading).
//
// Design (gfx950, wave64): a group of L lanes (L = E rounded up to a power of two,
// at most 64) owns one token; lane i holds experts i, i+L, i+2L, ... so the
// logits row is read with consecutive lanes on consecutive addresses.  Each
// candidate becomes a 64-bit key (order-preserving float bits << 32 | ~expert):
// the largest key is the largest logit, and among equal logits the lowest
// expert id.  k rounds of a butterfly max over the group pick the experts in
// order; the winner's owner drops it.  Gates are computed in fp64 by the first
// k lanes and rounded once to fp32.
#include <math.h>

#include "common.hpp"

namespace moe {

// Unsigned order of the keys equals the numeric order of the floats; -0.0 gets
// the key of +0.0 so that the two compare equal (IEEE equality).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

template <int L, int V>
__global__ void __launch_bounds__(256)
route_topk_kernel(const float* __restrict__ logits, int64_t tokens, int E, int k,
                  int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate) {
  constexpr int G = kWave / L;  // tokens per wave
  const int lane = lane_id();
  const int li = lane & (L - 1);
  const int gbase = lane & ~(L - 1);
  const int64_t wave = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;
  const int64_t nwaves = int64_t(gridDim.x) * (blockDim.x / kWave);
  for (int64_t t0 = wave * G; t0 < tokens; t0 += nwaves * G) {
    const int64_t t = t0 + lane / L;
    const bool tok_ok = t < tokens;
    uint64_t key[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = li + L * v;
      key[v] = 0ull;  // below every real key
      if (tok_ok && e < E) {
        const float f = logits[t * E + e];
        key[v] = (uint64_t(order_key(f)) << 32) | uint64_t(~uint32_t(e));
      }
    }
    int my_e = 0;
    float my_f = 0.0f;
    for (int j = 0; j < k; ++j) {
      uint64_t best = key[0];
#pragma unroll
      for (int v = 1; v < V; ++v) best = key[v] > best ? key[v] : best;
#pragma unroll
      for (int off = L / 2; off >= 1; off >>= 1) {
        const uint64_t o = __shfl_xor(best, off, kWave);
        best = o > best ? o : best;
      }
      const int e = int(~uint32_t(best));
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (li + L * v == e) key[v] = 0ull;
      if (li == j) {
        my_e = e;
        my_f = key_value(uint32_t(best >> 32));
      }
    }
    // Gates: g_j = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0), fp64, summed in
    // slot order, rounded once to fp32.
    const double l0 = double(__shfl(my_f, gbase, kWave));
    const double d = (li < k) ? exp(double(my_f) - l0) : 0.0;
    double s = 0.0;
    for (int j = 0; j < k; ++j) s += __shfl(d, gbase + j, kWave);
    if (tok_ok && li < k) {
      topk_idx[t * k + li] = my_e;
      topk_gate[t * k + li] = float(d / s);
    }
  }
}

template <int L, int V>
static hipError_t launch_route(const float* logits, int64_t tokens, int E, int k, int32_t* idx,
                               float* gate, hipStream_t stream) {
  constexpr int G = kWave / L;
  const int64_t per_block = 4 * G;
  int64_t blocks = (tokens + per_block - 1) / per_block;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL((route_topk_kernel<L, V>), dim3(unsigned(blocks)), dim3(256), 0, stream,
                     logits, tokens, E, k, idx, gate);
  return hipGetLastError();
}

hipError_t launch_route_topk(const float* logits, int64_t tokens, int E, int k, int32_t* idx,
                             float* gate, hipStream_t stream) {
  if (E <= 1) return launch_route<1, 1>(logits, tokens, E, k, idx, gate, stream);
  if (E <= 2) return launch_route<2, 1>(logits, tokens, E, k, idx, gate, stream);
  if (E <= 4) return launch_route<4, 1>(logits, tokens, E, k, idx, gate, stream);
  if (E <= 8) return launch_route<8, 1>(logits, tokens, E, k, idx, gate, stream);
  if (E <= 16) return launch_route<16, 1>(logits, tokens, E, k, idx, gate, stream);
  if (E <= 32) return launch_route<32, 1>(logits, tokens, E, k, idx, gate, stream);
  if (E <= 64) return launch_route<64, 1>(logits, tokens, E, k, idx, gate, stream);
  if (E <= 128) return launch_route<64, 2>(logits, tokens, E, k, idx, gate, stream);
  if (E <= 256) return launch_route<64, 4>(logits, tokens, E, k, idx, gate, stream);
  if (E <= 512) return launch_route<64, 8>(logits, tokens, E, k, idx, gate, stream);
  return launch_route<64, 16>(logits, tokens, E, k, idx, gate, stream);
}

}  // namespace moe
