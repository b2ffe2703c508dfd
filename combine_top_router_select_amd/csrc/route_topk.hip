// A1 - top-k routing with softmax gates over the selected logits.
//
// Source: "Expert Coupling in MoE Pretraining" (summary page), section
// "Background": every token goes to its k highest-scoring experts.  The gate is
// the softmax over the k selected logits (the pages speak of routing
// probabilities without a formula; this is the plainest reading).
//
// Design (gfx950, wave64): a group of L lanes owns one token (L = 16, or E
// rounded up to a power of two when E < 16), so a wave routes 64/L tokens at
// once; lane i holds experts i, i+L, i+2L, ..., so each logits load has
// consecutive lanes on consecutive addresses.  Each candidate becomes a 64-bit
// key (order-preserving float bits << 32 | ~expert): the largest key is the
// largest logit and, among equal logits, the lowest expert id.  Each of the k
// rounds takes the lane-local maximum, then the group maximum with a DPP
// butterfly inside the 16-lane row (quad permutes, half-row mirror, row mirror:
// no LDS round trip), and retires the winning key.  Lane j of the group keeps
// the round-j winner.  Gates are computed in fp64 (exp of the logit minus the
// largest one, divided by their DPP-summed total) and rounded once to fp32.
// FULL: the total runs over all E logits instead of the k selected ones
// (softmax over every expert, not renormalised over the selection).
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

// DPP lane permutations inside a 16-lane row.
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- 7 - i within each 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <- 15 - i within each 16 lanes

template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  return (uint64_t(dpp32<CTRL>(uint32_t(v >> 32))) << 32) | dpp32<CTRL>(uint32_t(v));
}

template <int CTRL>
__device__ __forceinline__ uint64_t max_step(uint64_t v) {
  const uint64_t o = dpp64<CTRL>(v);
  return o > v ? o : v;
}

template <int CTRL>
__device__ __forceinline__ double add_step(double v) {
  return v + __longlong_as_double((long long)dpp64<CTRL>(uint64_t(__double_as_longlong(v))));
}

// Maximum over the L-lane group (L <= 16, a power of two); every lane gets it.
template <int L>
__device__ __forceinline__ uint64_t group_max(uint64_t v) {
  if (L >= 2) v = max_step<kDppXor1>(v);
  if (L >= 4) v = max_step<kDppXor2>(v);
  if (L >= 8) v = max_step<kDppHalfMirror>(v);
  if (L >= 16) v = max_step<kDppMirror>(v);
  return v;
}

// Sum over the L-lane group in a fixed order; every lane gets it.
template <int L>
__device__ __forceinline__ double group_sum(double v) {
  if (L >= 2) v = add_step<kDppXor1>(v);
  if (L >= 4) v = add_step<kDppXor2>(v);
  if (L >= 8) v = add_step<kDppHalfMirror>(v);
  if (L >= 16) v = add_step<kDppMirror>(v);
  return v;
}

template <int L, int V, bool FULL>
__global__ void __launch_bounds__(256)
route_topk_kernel(const float* __restrict__ logits, int64_t tokens, int E, int k,
                  int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate) {
  constexpr int G = kWave / L;  // tokens per wave
  const int lane = lane_id();
  const int li = lane & (L - 1);
  const int64_t wave = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;
  const int64_t nwaves = int64_t(gridDim.x) * (blockDim.x / kWave);
  for (int64_t t0 = wave * G; t0 < tokens; t0 += nwaves * G) {
    const int64_t t = t0 + lane / L;
    const bool tok_ok = t < tokens;
    const int64_t tc = tok_ok ? t : tokens - 1;  // loads stay in bounds and unconditional
    float f[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = li + L * v;
      f[v] = logits[tc * E + (e < E ? e : E - 1)];
    }
    uint64_t key[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = li + L * v;
      key[v] = (tok_ok && e < E)
                   ? (uint64_t(order_key(f[v])) << 32) | uint64_t(~uint32_t(e))
                   : 0ull;  // below every real key
    }
    int my_e = 0;
    float my_f = 0.0f, l0 = 0.0f;
    for (int j = 0; j < k; ++j) {
      uint64_t best = key[0];
#pragma unroll
      for (int v = 1; v < V; ++v) best = key[v] > best ? key[v] : best;
      best = group_max<L>(best);
#pragma unroll
      for (int v = 0; v < V; ++v) key[v] = key[v] == best ? 0ull : key[v];
      const float f = key_value(uint32_t(best >> 32));
      if (j == 0) l0 = f;
      if (li == j) {
        my_e = int(~uint32_t(best));
        my_f = f;
      }
    }
    const double d = (li < k) ? exp(double(my_f) - double(l0)) : 0.0;
    double part = d;
    if (FULL) {
      part = 0.0;
#pragma unroll
      for (int v = 0; v < V; ++v)
        part += (li + L * v < E) ? exp(double(f[v]) - double(l0)) : 0.0;
    }
    const double s = group_sum<L>(part);
    if (tok_ok && li < k) {
      topk_idx[t * k + li] = my_e;
      topk_gate[t * k + li] = float(d / s);
    }
  }
}

template <int L, int V, bool FULL>
static hipError_t launch_route(const float* logits, int64_t tokens, int E, int k, int32_t* idx,
                               float* gate, hipStream_t stream) {
  constexpr int G = kWave / L;
  const int64_t per_block = 4 * G;
  int64_t blocks = (tokens + per_block - 1) / per_block;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL((route_topk_kernel<L, V, FULL>), dim3(unsigned(blocks)), dim3(256), 0, stream,
                     logits, tokens, E, k, idx, gate);
  return hipGetLastError();
}

template <bool FULL>
static hipError_t launch_route_e(const float* logits, int64_t tokens, int E, int k, int32_t* idx,
                                 float* gate, hipStream_t stream) {
  if (E <= 1) return launch_route<1, 1, FULL>(logits, tokens, E, k, idx, gate, stream);
  if (E <= 2) return launch_route<2, 1, FULL>(logits, tokens, E, k, idx, gate, stream);
  if (E <= 4) return launch_route<4, 1, FULL>(logits, tokens, E, k, idx, gate, stream);
  if (E <= 8) return launch_route<8, 1, FULL>(logits, tokens, E, k, idx, gate, stream);
  if (E <= 16) return launch_route<16, 1, FULL>(logits, tokens, E, k, idx, gate, stream);
  if (E <= 32) return launch_route<16, 2, FULL>(logits, tokens, E, k, idx, gate, stream);
  if (E <= 64) return launch_route<16, 4, FULL>(logits, tokens, E, k, idx, gate, stream);
  if (E <= 128) return launch_route<16, 8, FULL>(logits, tokens, E, k, idx, gate, stream);
  if (E <= 256) return launch_route<16, 16, FULL>(logits, tokens, E, k, idx, gate, stream);
  if (E <= 512) return launch_route<16, 32, FULL>(logits, tokens, E, k, idx, gate, stream);
  return launch_route<16, 64, FULL>(logits, tokens, E, k, idx, gate, stream);
}

// full_softmax: gates are the softmax over all E logits at the selected
// experts; otherwise the softmax over the k selected logits.
hipError_t launch_route_topk(const float* logits, int64_t tokens, int E, int k, int full_softmax,
                             int32_t* idx, float* gate, hipStream_t stream) {
  if (full_softmax) return launch_route_e<true>(logits, tokens, E, k, idx, gate, stream);
  return launch_route_e<false>(logits, tokens, E, k, idx, gate, stream);
}

}  // namespace moe
