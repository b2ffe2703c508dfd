// Shared device helpers for the gfx950 (CDNA4) kernels: wave64 lane masks,
// broadcasts, 16-byte vector loads/stores and the plan layout that
// moe_send_counts leaves in the workspace for the dispatch kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;          // CDNA wavefront width
// Tokens per plan tile, one routing workgroup (16, 32 or 64 compile).  Measured
// at 4096 tokens, top-6 of 64, one stream, per step: 16 -> 44.6 us, 32 -> 44.0,
// 64 -> 44.75; with two streams 40.7, 40.0, 39.9.  Smaller tiles spread the
// routing over more CUs (at 16: 3.26 us per call against 3.36 at 32 and 4.30
// at 64) but give the dispatch 2x / 4x more plan entries to look up, which
// costs it 0.15 / 0.5 us.
constexpr int kTile = 32;
constexpr int kWaveTile = 64;      // tokens per counting wave and per co-selection bitmap
constexpr int kTilesPerWave = kWaveTile / kTile;
static_assert(kTile == 16 || kTile == 32 || kTile == 64, "plan tiles of 16, 32 or 64 tokens");

// A bitmap of one plan tile's tokens, and the piece of a 64-token co-selection
// bitmap that one tile fills.
template <int N> struct TileBits;
template <> struct TileBits<16> { typedef uint32_t mask; typedef uint16_t piece; };
template <> struct TileBits<32> { typedef uint32_t mask; typedef uint32_t piece; };
template <> struct TileBits<64> { typedef uint64_t mask; typedef uint64_t piece; };
typedef TileBits<kTile>::mask TileMask;
typedef TileBits<kTile>::piece TilePiece;
constexpr uint32_t kNoSlot = 0xFFFFFFFFu;  // plan code of an empty slot (received rows)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = __lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Wave-uniform value of `v` held by lane `src` (src must be wave-uniform).
__device__ __forceinline__ int bcast(int v, int src) {
  return __builtin_amdgcn_readlane(v, src);
}
__device__ __forceinline__ float bcastf(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void store16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ void store16_nt(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ u32x4 load16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// Sum of the 16 bytes of v (v_sad_u8 against zero adds four bytes at a time).
__device__ __forceinline__ int byte_sum(const u32x4& v) {
  uint32_t s = __builtin_amdgcn_sad_u8(v.x, 0u, 0u);
  s = __builtin_amdgcn_sad_u8(v.y, 0u, s);
  s = __builtin_amdgcn_sad_u8(v.z, 0u, s);
  s = __builtin_amdgcn_sad_u8(v.w, 0u, s);
  return int(s);
}

// Keeps the first n bytes of v and zeroes the rest (n <= 0: all zero).
__device__ __forceinline__ u32x4 keep_bytes(u32x4 v, int n) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int nb = clampi(n - 4 * i, 0, 4);
    const uint32_t mk = nb >= 4 ? ~0u : ((1u << (8 * nb)) - 1u);
    r[i] = v[i] & mk;
  }
  return r;
}

// Plan written by moe_send_counts, read by the dispatch kernels.  A plan tile
// is kTile consecutive tokens.  Per-column arrays are column-major with the tile
// index padded to Bp = roundup(B, 16), so that a column's tile counts come in
// 16-byte vectors of 16 tiles.
//   header[0]        total rows (N, or D in dedup mode)
//   gbase[CP][Bp/16] int32: first row, in the send buffer, of each group of 16
//                    tiles of position column c (the expert in plain mode, the
//                    rank in dedup mode)
//   tcnt[C][Bp]      uint8: tokens of tile b that use column c (experts, then
//                    ranks in dedup mode); at most 64, the tile size
//   lslot[T][k]      uint32: (position column << 8) | rank of (t, j) among the
//                    tile's earlier tokens that use the same position column
//   ctot[C]          int32: column totals (large plans, whose scan runs as two
//                    many-workgroup kernels)
//   bm[BW][E]        uint64, BW = ceil(T / 64): bit i set when token i of the
//                    64-token block selects expert e (written by both counting
//                    paths, read by the co-selection counts)
// The row of (t, j) is gbase[c][b / 16] + (counts of tiles 16 (b / 16) .. b - 1
// in column c) + rank, with b = t / kTile.
struct PlanLayout {
  int64_t tiles;      // B = ceil(T / kTile)
  int64_t tiles_pad;  // Bp = roundup(B, 16)
  int64_t groups;     // Bp / 16
  int cols;           // C: columns counted per tile (experts, + ranks in dedup mode)
  int pos_cols;       // CP: position columns (experts, or ranks in dedup mode)
  int cbase;          // tcnt column of position column 0 (E in dedup mode, else 0)
  int64_t bm_tiles;   // BW = ceil(T / 64): 64-token blocks of the expert bitmaps
  size_t base_off;    // byte offsets inside the workspace
  size_t tcnt_off;
  size_t lslot_off;
  size_t ctot_off;
  size_t bm_off;
  size_t bytes;
};

__host__ __device__ inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

__host__ __device__ inline PlanLayout plan_layout(int64_t tokens, int n_experts, int top_k,
                                                  int n_ranks, int dedup) {
  PlanLayout p;
  p.tiles = (tokens + kTile - 1) / kTile;
  p.tiles_pad = (p.tiles + 15) / 16 * 16;
  p.groups = p.tiles_pad / 16;
  p.cols = n_experts + (dedup ? n_ranks : 0);
  p.pos_cols = dedup ? n_ranks : n_experts;
  p.cbase = dedup ? n_experts : 0;
  p.bm_tiles = (tokens + kWaveTile - 1) / kWaveTile;
  p.base_off = 256;
  p.tcnt_off = align256(p.base_off + size_t(p.pos_cols) * size_t(p.groups) * 4);
  p.lslot_off = align256(p.tcnt_off + size_t(p.cols) * size_t(p.tiles_pad));
  p.ctot_off = align256(p.lslot_off + size_t(tokens) * size_t(top_k) * 4);
  p.bm_off = align256(p.ctot_off + size_t(p.cols) * 4);
  p.bytes = align256(p.bm_off + size_t(p.bm_tiles) * size_t(n_experts) * 8);
  return p;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and row
// broadcasts (the gfx9 family has row_bcast:15/31): no LDS round trips.
__device__ __forceinline__ int wave_incl_scan(int x) {
  int v = x + __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);         // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, x, 0x113, 0xF, 0xF, true);         // row_shr:3
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xE, false);        // row_shr:4, lanes 4..15
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xC, false);        // row_shr:8, lanes 8..15
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);        // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);        // row_bcast:31 -> rows 2, 3
  return v;
}

// Keeps the compiler from moving LDS accesses of one wave across this point;
// a wave's own LDS operations are executed in program order.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

}  // namespace moe
