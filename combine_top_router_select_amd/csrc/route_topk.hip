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
// consecutive lanes on consecutive addresses.  Each candidate's key is its
// logit's order-preserving 32-bit pattern.  Each of the k rounds takes the
// lane-local maximum, the group maximum with DPP inside the 16-lane row (quad
// permutes, half-row mirror, row mirror: no LDS round trip), then the group
// minimum of the expert ids holding that key (the lowest id wins a tie), and
// retires that candidate.  Lane j of the group keeps the round-j winner.
// Gates are computed in fp64 (exp of the logit minus the largest one, divided
// by their DPP-summed total) and rounded once to fp32.
// FULL: the total runs over all E logits instead of the k selected ones
// (softmax over every expert, not renormalised over the selection).
#include "route_tile.hpp"

namespace moe {

template <int L, int V, int VEC, bool FULL>
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
    RouteSlots<L> r;
    route_token<L, V, VEC, FULL>(logits, tokens, E, k, t, tok_ok, li, r);
#pragma unroll
    for (int s = 0; s < RouteSlots<L>::N; ++s) {
      const int j = li + L * s;
      if (tok_ok && j < k) {
        topk_idx[t * k + j] = r.e[s];
        topk_gate[t * k + j] = float(r.num[s] / r.den);
      }
    }
  }
}

// The fused routing kernel: one workgroup per plan tile (route_tile_block).
template <int L, int V, int VEC, bool FULL, bool DEDUP>
__global__ void __launch_bounds__(kTile * L)
route_tile_kernel(const float* __restrict__ logits, int64_t tokens, int E, int k, int R,
                  const int32_t* __restrict__ place, int m, int64_t Bp,
                  int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
                  uint8_t* __restrict__ tcnt, uint32_t* __restrict__ lslot,
                  TilePiece* __restrict__ bm) {
  extern __shared__ TileMask s_rdyn[];
  route_tile_block<L, V, VEC, FULL, DEDUP>(logits, tokens, E, k, R, place, m, Bp, topk_idx,
                                           topk_gate, tcnt, lslot, bm, blockIdx.x, s_rdyn);
}

template <int L, int V, int VEC, bool FULL>
static hipError_t launch_route(const float* logits, int64_t tokens, int E, int k, int32_t* idx,
                               float* gate, hipStream_t stream) {
  constexpr int G = kWave / L;
  const int64_t per_block = 4 * G;
  int64_t blocks = (tokens + per_block - 1) / per_block;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL((route_topk_kernel<L, V, VEC, FULL>), dim3(unsigned(blocks)), dim3(256), 0,
                     stream, logits, tokens, E, k, idx, gate);
  return hipGetLastError();
}

// Lanes per token L = min(16, E rounded up to a power of two) and logits per
// lane V = ceil(E / L).  (Four lanes with 16 logits each were measured slower
// at E = 64: one wave per SIMD then leaves the round's dependent chain
// unhidden.)  VEC = 4 needs V % 4 == 0.
template <bool FULL, int VEC>
static hipError_t launch_route_v(const float* logits, int64_t tokens, int E, int k, int32_t* idx,
                                 float* gate, hipStream_t st) {
  if (E <= 64) return launch_route<16, 4, VEC, FULL>(logits, tokens, E, k, idx, gate, st);
  if (E <= 128) return launch_route<16, 8, VEC, FULL>(logits, tokens, E, k, idx, gate, st);
  if (E <= 256) return launch_route<16, 16, VEC, FULL>(logits, tokens, E, k, idx, gate, st);
  if (E <= 512) return launch_route<16, 32, VEC, FULL>(logits, tokens, E, k, idx, gate, st);
  return launch_route<16, 64, VEC, FULL>(logits, tokens, E, k, idx, gate, st);
}

template <bool FULL>
static hipError_t launch_route_small(const float* logits, int64_t tokens, int E, int k,
                                     int32_t* idx, float* gate, hipStream_t st) {
  if (E <= 1) return launch_route<1, 1, 1, FULL>(logits, tokens, E, k, idx, gate, st);
  if (E <= 2) return launch_route<2, 1, 1, FULL>(logits, tokens, E, k, idx, gate, st);
  if (E <= 4) return launch_route<4, 1, 1, FULL>(logits, tokens, E, k, idx, gate, st);
  if (E <= 8) return launch_route<8, 1, 1, FULL>(logits, tokens, E, k, idx, gate, st);
  if (E <= 16) return launch_route<16, 1, 1, FULL>(logits, tokens, E, k, idx, gate, st);
  return launch_route<16, 2, 1, FULL>(logits, tokens, E, k, idx, gate, st);
}

template <bool FULL>
static hipError_t launch_route_e(const float* logits, int64_t tokens, int E, int k, int32_t* idx,
                                 float* gate, hipStream_t stream) {
  if (E <= 32) return launch_route_small<FULL>(logits, tokens, E, k, idx, gate, stream);
  if (E % 4 == 0) return launch_route_v<FULL, 4>(logits, tokens, E, k, idx, gate, stream);
  return launch_route_v<FULL, 1>(logits, tokens, E, k, idx, gate, stream);
}

// full_softmax: gates are the softmax over all E logits at the selected
// experts; otherwise the softmax over the k selected logits.
hipError_t launch_route_topk(const float* logits, int64_t tokens, int E, int k, int full_softmax,
                             int32_t* idx, float* gate, hipStream_t stream) {
  if (tokens == 0) return hipSuccess;  // no grid to launch
  if (full_softmax) return launch_route_e<true>(logits, tokens, E, k, idx, gate, stream);
  return launch_route_e<false>(logits, tokens, E, k, idx, gate, stream);
}

hipError_t launch_plan_scan(int64_t T, int E, int k, int R, const int32_t* place, int dedup,
                            int32_t* expert_counts, int32_t* rank_counts, int32_t* rank_offsets,
                            int32_t* expert_offsets, void* workspace, hipStream_t stream);
hipError_t launch_send_counts(const int32_t* idx, int64_t T, int E, int k, int R,
                              const int32_t* place, int dedup, int32_t* expert_counts,
                              int32_t* rank_counts, int32_t* rank_offsets,
                              int32_t* expert_offsets, void* workspace, hipStream_t stream);

// Largest expert count and token count routed by the fused kernel; beyond them
// the routing and the counting run as separate kernels (same results).
constexpr int kFusedMaxExperts = 256;
constexpr int64_t kFusedMaxTokens = int64_t(1) << 24;

template <int L, int V, int VEC, bool FULL>
static hipError_t launch_route_tile(const float* logits, int64_t T, int E, int k, int R,
                                    const int32_t* place, int dedup, int32_t* idx, float* gate,
                                    void* workspace, hipStream_t stream) {
  const PlanLayout pl = plan_layout(T, E, k, R, dedup);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* tcnt = ws + pl.tcnt_off;
  uint32_t* lslot = reinterpret_cast<uint32_t*>(ws + pl.lslot_off);
  TilePiece* bm = reinterpret_cast<TilePiece*>(ws + pl.bm_off);
  const size_t lds = route_tile_lds(pl.cols, E);
  if (dedup)
    hipLaunchKernelGGL((route_tile_kernel<L, V, VEC, FULL, true>), dim3(unsigned(pl.tiles)),
                       dim3(kTile * L), lds, stream, logits, T, E, k, R, place, E / R,
                       pl.tiles_pad, idx, gate, tcnt, lslot, bm);
  else
    hipLaunchKernelGGL((route_tile_kernel<L, V, VEC, FULL, false>), dim3(unsigned(pl.tiles)),
                       dim3(kTile * L), lds, stream, logits, T, E, k, R, place, E / R,
                       pl.tiles_pad, idx, gate, tcnt, lslot, bm);
  return hipGetLastError();
}

template <bool FULL, int VEC>
static hipError_t launch_route_tile_e(const float* logits, int64_t T, int E, int k, int R,
                                      const int32_t* place, int dedup, int32_t* idx, float* gate,
                                      void* ws, hipStream_t st) {
#define MOE_RT(LL, VV, VC) \
  launch_route_tile<LL, VV, VC, FULL>(logits, T, E, k, R, place, dedup, idx, gate, ws, st)
  if (E <= 1) return MOE_RT(1, 1, 1);
  if (E <= 2) return MOE_RT(2, 1, 1);
  if (E <= 4) return MOE_RT(4, 1, 1);
  if (E <= 8) return MOE_RT(8, 1, 1);
  if (E <= 16) return MOE_RT(16, 1, 1);
  if (E <= 32) return MOE_RT(16, 2, 1);
  if (E <= 64) return MOE_RT(16, 4, VEC);
  if (E <= 128) return MOE_RT(16, 8, VEC);
  return MOE_RT(16, 16, VEC);
#undef MOE_RT
}

hipError_t launch_coselect_bm(const uint64_t* bm, int64_t cs_tokens, int E, int32_t* W,
                              hipStream_t stream);

// Whether the fused routing kernel takes this shape.
bool route_tiles_fit(int64_t T, int E) { return T > 0 && E <= kFusedMaxExperts && T <= kFusedMaxTokens; }

// The fused routing kernel alone (routing, tile counts, slot codes, bitmaps):
// the plan without its scan, for a dispatch that scans it itself.  Only for
// shapes that route_tiles_fit() accepts.
hipError_t launch_route_tiles(const float* logits, int64_t T, int E, int k, int full_softmax,
                              int R, const int32_t* place, int dedup, int32_t* idx, float* gate,
                              void* workspace, hipStream_t stream) {
  const bool v4 = E % 4 == 0;
#define MOE_RTE(FU, VC) \
  launch_route_tile_e<FU, VC>(logits, T, E, k, R, place, dedup, idx, gate, workspace, stream)
  return full_softmax ? (v4 ? MOE_RTE(true, 4) : MOE_RTE(true, 1))
                      : (v4 ? MOE_RTE(false, 4) : MOE_RTE(false, 1));
#undef MOE_RTE
}

// Routing, the dispatch plan and (W non-null) the co-selection counts of the
// first cs_tokens tokens: the fused kernel then the scan, or (large E or T)
// the routing kernel, the counting kernel and the scan; then the co-selection
// counts from the 64-token expert bitmaps that either path leaves in the plan.
hipError_t launch_route_plan(const float* logits, int64_t T, int E, int k, int full_softmax,
                             int R, const int32_t* place, int dedup, int32_t* idx, float* gate,
                             int32_t* expert_counts, int32_t* rank_counts, int32_t* rank_offsets,
                             int32_t* expert_offsets, int64_t cs_tokens, int32_t* W,
                             void* workspace, hipStream_t stream) {
  hipError_t err;
  if (E > kFusedMaxExperts || T > kFusedMaxTokens) {
    err = launch_route_topk(logits, T, E, k, full_softmax, idx, gate, stream);
    if (err != hipSuccess) return err;
    err = launch_send_counts(idx, T, E, k, R, place, dedup, expert_counts, rank_counts,
                             rank_offsets, expert_offsets, workspace, stream);
  } else {
    if (T > 0) {
      const bool v4 = E % 4 == 0;
#define MOE_RTE(FU, VC) \
  launch_route_tile_e<FU, VC>(logits, T, E, k, R, place, dedup, idx, gate, workspace, stream)
      err = full_softmax ? (v4 ? MOE_RTE(true, 4) : MOE_RTE(true, 1))
                         : (v4 ? MOE_RTE(false, 4) : MOE_RTE(false, 1));
#undef MOE_RTE
      if (err != hipSuccess) return err;
    }
    err = launch_plan_scan(T, E, k, R, place, dedup, expert_counts, rank_counts, rank_offsets,
                           expert_offsets, workspace, stream);
  }
  if (err != hipSuccess || W == nullptr || cs_tokens <= 0) return err;
  const PlanLayout pl = plan_layout(T, E, k, R, dedup);
  const uint64_t* bm =
      reinterpret_cast<const uint64_t*>(static_cast<const uint8_t*>(workspace) + pl.bm_off);
  return launch_coselect_bm(bm, cs_tokens, E, W, stream);
}

}  // namespace moe
