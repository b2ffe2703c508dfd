// Top-k routing of a token by a group of L lanes, and the routing of one
// plan tile with its tile counts, slot codes and expert bitmaps by one
// workgroup: device routines of the routing kernels (route_topk.hip) and of
// the combine that also routes the next batch (combine_route.hip).  The
// method and the design are described in route_topk.hip.
#pragma once

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
// stay in bounds (token tokens - 1) and the results are unused.  full (or
// FULL): the gate denominator runs over all E logits.
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
                                            RouteSlots<L>& out, bool full = false) {
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
  if (FULL || full) {
    part = 0.0;
#pragma unroll
    for (int v = 0; v < V; ++v)
      part += expert_of<L, VEC>(li, v) < E ? exp(double(f[v]) - l0) : 0.0;
  }
  out.den = group_sum<L>(part);
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
// the co-selection counts are taken from there later, by workgroups of the
// dispatch launch or by a kernel of their own (done here, they would cost one
// atomic add per co-selected pair and tile).

// LDS bytes of route_tile_block: C = E (+ R in dedup mode) TileMasks and E
// ints.
__host__ __device__ inline size_t route_tile_lds(int C, int E) {
  return size_t(C) * sizeof(TileMask) + size_t(E) * sizeof(int32_t);
}

// Plan tile b routed by the calling workgroup of kTile * L threads; s_rdyn:
// route_tile_lds() bytes of LDS.  DEDUP or dedup: dedup mode; FULL or full:
// the softmax over all E logits (runtime flags for callers that host one
// routing variant for every mode).
template <int L, int V, int VEC, bool FULL, bool DEDUP>
__device__ __forceinline__ void route_tile_block(
    const float* __restrict__ logits, int64_t tokens, int E, int k, int R,
    const int32_t* __restrict__ place, int m, int64_t Bp, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_gate, uint8_t* __restrict__ tcnt, uint32_t* __restrict__ lslot,
    TilePiece* __restrict__ bm, int64_t b, TileMask* s_rdyn, bool full = false,
    bool dedup = false) {
  constexpr int NS = RouteSlots<L>::N;
  const bool dd = DEDUP || dedup;
  const int C = E + (dd ? R : 0);
  TileMask* bits = s_rdyn;                                     // [C]
  int32_t* s_rank = reinterpret_cast<int32_t*>(s_rdyn + C);   // [E] (dedup, explicit placement)
  const int tid = threadIdx.x;
  const int nthreads = kTile * L;
  const int li = lane_id() & (L - 1);
  const int tl = tid / L;  // token within the tile
  const int64_t t = b * kTile + tl;
  const bool tok_ok = t < tokens;
  for (int c = tid; c < C; c += nthreads) bits[c] = 0;
  const bool has_rank = dd && place;
  if (has_rank)
    for (int e = tid; e < E; e += nthreads) s_rank[e] = clampi(place[e], 0, R - 1);
  RouteSlots<L> r;
  route_token<L, V, VEC, FULL>(logits, tokens, E, k, t, tok_ok, li, r, full);
  __syncthreads();  // bitmaps cleared, ranks loaded
  const TileMask bit = TileMask(1) << tl;
  int col[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int j = li + L * s;
    const bool mine = tok_ok && j < k;
    const int e = mine ? r.e[s] : 0;  // slots without a selection keep an in-range id
    col[s] = dd ? (has_rank ? s_rank[e] : e / m) : e;
    if (mine) {
      topk_idx[t * k + j] = e;
      topk_gate[t * k + j] = float(r.num[s] / r.den);
      lds_or(&bits[e], bit);
      if (dd) lds_or(&bits[E + col[s]], bit);
    }
  }
  __syncthreads();
  const TileMask below = bit - 1;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int j = li + L * s;
    if (tok_ok && j < k) {
      const TileMask mb = bits[dd ? E + col[s] : col[s]];
      lslot[t * k + j] = (uint32_t(col[s]) << 8) | uint32_t(__popcll(uint64_t(mb & below)));
    }
  }
  for (int c = tid; c < C; c += nthreads) tcnt[c * Bp + b] = uint8_t(__popcll(uint64_t(bits[c])));
  // piece b % kTilesPerWave of the 64-token block b / kTilesPerWave
  // (little-endian pieces)
  for (int e = tid; e < E; e += nthreads)
    bm[((b / kTilesPerWave) * E + e) * kTilesPerWave + b % kTilesPerWave] = TilePiece(bits[e]);
}

}  // namespace moe
