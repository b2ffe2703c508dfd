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

// Maximum / minimum of 32-bit values over the L-lane group; every lane gets it.
template <int L>
__device__ __forceinline__ uint32_t group_max32(uint32_t v) {
  if (L >= 2) v = max(v, dpp32<kDppXor1>(v));
  if (L >= 4) v = max(v, dpp32<kDppXor2>(v));
  if (L >= 8) v = max(v, dpp32<kDppHalfMirror>(v));
  if (L >= 16) v = max(v, dpp32<kDppMirror>(v));
  return v;
}

template <int L>
__device__ __forceinline__ uint32_t group_min32(uint32_t v) {
  if (L >= 2) v = min(v, dpp32<kDppXor1>(v));
  if (L >= 4) v = min(v, dpp32<kDppXor2>(v));
  if (L >= 8) v = min(v, dpp32<kDppHalfMirror>(v));
  if (L >= 16) v = min(v, dpp32<kDppMirror>(v));
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

constexpr int kMaxTopK = 16;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Expert held by lane li of a group in its v-th register: VEC consecutive
// experts per lane and chunk, chunks of L * VEC experts.  Ascending v is
// ascending expert id within a lane.
template <int L, int VEC>
__device__ __forceinline__ int expert_of(int li, int v) {
  return (v / VEC) * (L * VEC) + li * VEC + (v % VEC);
}

// Winner slots kept by one lane: rounds li, li + L, li + 2L, ... of its group.
template <int L>
struct RouteSlots {
  static constexpr int N = (kMaxTopK + L - 1) / L;
  int e[N];          // expert id of round li + L s
  double num[N];     // its gate numerator exp(l - l_max), fp64
  double den;        // the group's gate denominator
};

// Routes token t with one group of L lanes (li = lane within the group); V
// logits per lane (VEC = 4: 16-byte loads, E % 4 == 0).  tok_ok false: loads
// stay in bounds (token tokens - 1) and the results are unused.
//
// Selection with 32-bit operations only: candidate keys are the order keys of
// the logits, raised to at least 1 so that 0 marks retired and absent
// candidates (only the NaN pattern 0xFFFFFFFF has order key 0, and NaN logits
// are outside the contract).  A round takes the group maximum of the keys,
// then the group minimum of the expert ids holding it (the lowest id wins a
// tie), and retires that candidate; each group reduction is log2(L) DPP
// max/min steps.  Every lane of the group sees every round's winner; lane li
// keeps rounds li + L s.  The rounds are unrolled, so slot indices are static.
template <int L, int V, int VEC, bool FULL>
__device__ __forceinline__ void route_token(const float* __restrict__ logits, int64_t tokens,
                                            int E, int k, int64_t t, bool tok_ok, int li,
                                            RouteSlots<L>& out) {
  const int64_t tc = tok_ok ? t : tokens - 1;  // loads stay in bounds and unconditional
  const float* row = logits + tc * E;
  float f[V];
  if (VEC == 4) {
#pragma unroll
    for (int c = 0; c < V / 4; ++c) {
      const int base = c * L * 4 + li * 4;
      const f32x4 q = *reinterpret_cast<const f32x4*>(row + (base <= E - 4 ? base : E - 4));
#pragma unroll
      for (int i = 0; i < 4; ++i) f[4 * c + i] = q[i];
    }
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = expert_of<L, VEC>(li, v);
      f[v] = row[e < E ? e : E - 1];
    }
  }
  uint32_t key[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const uint32_t ok = order_key(f[v]);
    key[v] = (tok_ok && expert_of<L, VEC>(li, v) < E) ? (ok > 1u ? ok : 1u) : 0u;
  }
  uint32_t my_key[RouteSlots<L>::N];
  uint32_t key0 = 0u;
#pragma unroll
  for (int s = 0; s < RouteSlots<L>::N; ++s) {
    out.e[s] = 0;
    my_key[s] = 0u;
  }
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j >= k) continue;  // uniform; every round is its own unrolled copy
    uint32_t m = key[0];
#pragma unroll
    for (int v = 1; v < V; ++v) m = key[v] > m ? key[v] : m;
    const uint32_t best = group_max32<L>(m);
    uint32_t cand = 0xFFFFFFFFu;  // lowest expert id of this lane holding the maximum
#pragma unroll
    for (int v = V - 1; v >= 0; --v)
      cand = key[v] == best ? uint32_t(expert_of<L, VEC>(li, v)) : cand;
    const uint32_t win = group_min32<L>(cand);
#pragma unroll
    for (int v = 0; v < V; ++v) key[v] = uint32_t(expert_of<L, VEC>(li, v)) == win ? 0u : key[v];
    if (j == 0) key0 = best;
    if (li == j % L) {
      out.e[j / L] = int(win);
      my_key[j / L] = best;
    }
  }
  const double l0 = double(key_value(key0));
  double part = 0.0;
#pragma unroll
  for (int s = 0; s < RouteSlots<L>::N; ++s) {
    out.num[s] = li + L * s < k ? exp(double(key_value(my_key[s])) - l0) : 0.0;
    part += out.num[s];
  }
  if (FULL) {
    part = 0.0;
#pragma unroll
    for (int v = 0; v < V; ++v)
      part += expert_of<L, VEC>(li, v) < E ? exp(double(f[v]) - l0) : 0.0;
  }
  out.den = group_sum<L>(part);
}

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

__device__ __forceinline__ void lds_or(uint32_t* p, uint32_t v) { atomicOr(p, v); }
__device__ __forceinline__ void lds_or(uint64_t* p, uint64_t v) {
  atomicOr(reinterpret_cast<unsigned long long*>(p), static_cast<unsigned long long>(v));
}

// Routing fused with the per-tile counts of the dispatch plan: one workgroup
// per plan tile of kTile = 32 tokens, L lanes per token (32 L threads; at
// T = 4096 and L = 16, 128 workgroups of 512 threads).  Each selected expert
// sets its token's bit in an LDS bitmap of its column (the expert; in dedup
// mode also its rank),
// after which the popcount of the bits below the token is its rank in the tile
// and the popcount of the whole bitmap is the tile's count - the same plan
// entries as the separate counting kernel writes from topk_idx.  Saves that
// kernel's launch and its reread of the ids.  The expert bitmaps also go to
// the plan's 64-token co-selection bitmaps (bm), as this tile's piece of them;
// the co-selection counts are taken from there by a later kernel (done here,
// they would cost one atomic add per co-selected pair and tile).
template <int L, int V, int VEC, bool FULL, bool DEDUP>
__global__ void __launch_bounds__(kTile * L)
route_tile_kernel(const float* __restrict__ logits, int64_t tokens, int E, int k, int R,
                  const int32_t* __restrict__ place, int m, int64_t Bp,
                  int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
                  uint8_t* __restrict__ tcnt, uint32_t* __restrict__ lslot,
                  TilePiece* __restrict__ bm) {
  extern __shared__ TileMask s_rdyn[];
  constexpr int NS = RouteSlots<L>::N;
  const int C = E + (DEDUP ? R : 0);
  TileMask* bits = s_rdyn;                                     // [C]
  int32_t* s_rank = reinterpret_cast<int32_t*>(s_rdyn + C);   // [E] (dedup, explicit placement)
  const int tid = threadIdx.x;
  const int nthreads = kTile * L;
  const int64_t b = blockIdx.x;
  const int li = lane_id() & (L - 1);
  const int tl = tid / L;  // token within the tile
  const int64_t t = b * kTile + tl;
  const bool tok_ok = t < tokens;
  for (int c = tid; c < C; c += nthreads) bits[c] = 0;
  const bool has_rank = DEDUP && place;
  if (has_rank)
    for (int e = tid; e < E; e += nthreads) s_rank[e] = clampi(place[e], 0, R - 1);
  RouteSlots<L> r;
  route_token<L, V, VEC, FULL>(logits, tokens, E, k, t, tok_ok, li, r);
  __syncthreads();  // bitmaps cleared, ranks loaded
  const TileMask bit = TileMask(1) << tl;
  int col[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int j = li + L * s;
    const bool mine = tok_ok && j < k;
    const int e = mine ? r.e[s] : 0;  // slots without a selection keep an in-range id
    col[s] = DEDUP ? (has_rank ? s_rank[e] : e / m) : e;
    if (mine) {
      topk_idx[t * k + j] = e;
      topk_gate[t * k + j] = float(r.num[s] / r.den);
      lds_or(&bits[e], bit);
      if (DEDUP) lds_or(&bits[E + col[s]], bit);
    }
  }
  __syncthreads();
  const TileMask below = bit - 1;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int j = li + L * s;
    if (tok_ok && j < k) {
      const TileMask mb = bits[DEDUP ? E + col[s] : col[s]];
      lslot[t * k + j] = (uint32_t(col[s]) << 8) | uint32_t(__popcll(uint64_t(mb & below)));
    }
  }
  for (int c = tid; c < C; c += nthreads) tcnt[c * Bp + b] = uint8_t(__popcll(uint64_t(bits[c])));
  // piece b % kTilesPerWave of the 64-token block b / kTilesPerWave
  // (little-endian pieces)
  for (int e = tid; e < E; e += nthreads)
    bm[((b / kTilesPerWave) * E + e) * kTilesPerWave + b % kTilesPerWave] = TilePiece(bits[e]);
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
  const size_t lds = size_t(pl.cols) * sizeof(TileMask) + size_t(E) * sizeof(int32_t);
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
