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
// Counting a 64-token tile (one wave, one lane per token): every column
// (expert; in dedup mode also rank) gets a 64-bit LDS bitmap of the tile's
// tokens that use it, built with ds_or_b64 (order independent).  popcount of
// the bits below a lane is the token's rank among the tile's earlier users of
// the column; popcount of the whole bitmap is the tile's count.  The tile
// counts are then scanned over tiles, per column, into the absolute first row
// of each tile in each column.  A row's position is base[column][tile] + rank,
// which makes the send buffer order (rank, expert, token) - or (rank, token) -
// stable and deterministic.  No global atomics anywhere.
//
// Two kernels: tile_counts (one wave per tile, so the per-assignment work and
// its memory traffic spread over many CUs) and plan_scan (one workgroup, which
// only reads the per-tile counts, one byte each, and writes the bases).  Both
// per-tile arrays are column-major, so a scan thread streams a run of one
// column's tiles with 16-byte loads and stores.
//
// All global loads are issued unconditionally from clamped, in-bounds
// addresses and only stores are predicated: a load under a branch is followed
// by a wait for it, which would serialise them.
#include "common.hpp"
#include "moe_route.h"

namespace moe {

// floor(f / k) for 0 <= f < 2^24 and 2 <= k <= 16 is __umulhi(f, ceil(2^32 / k)):
// the rounding error of the reciprocal, below f / 2^32, never reaches 1/k.
__host__ __device__ inline uint32_t kdiv_mul(int k) {
  return k <= 1 ? 0u : uint32_t(((1ull << 32) + uint64_t(k) - 1) / uint64_t(k));
}
__device__ __forceinline__ int kdiv(uint32_t f, uint32_t mul, int k) {
  return k == 1 ? int(f) : int(__umulhi(f, mul));
}

// Raw ids of one tile for the calling wave: lane l takes the tile's flat id
// positions l, l + 64, ... (each load covers 256 contiguous bytes).  Positions
// past the end read the last id instead (no branch, no out-of-bounds access);
// callers clamp values where they use them, so that a prefetch does not wait
// for its own loads.
template <int KMAX>
__device__ __forceinline__ void load_tile_ids(int (&raw)[KMAX], const int32_t* __restrict__ idx,
                                              int64_t f0, int64_t total, int lane) {
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    const int64_t f = f0 + lane + kWave * r;
    raw[r] = idx[f < total ? f : total - 1];
  }
}

// Counts one 64-token tile in the calling wave.  `bits` holds C zeroed
// bitmaps: column c's bit i is set when token i of the tile uses column c.
// Lane l owns the ids at flat positions l + 64 r of the tile (token
// (l + 64 r) / k, slot (l + 64 r) % k) and writes their slot codes back at the
// same positions, so loads and stores stay coalesced.  In dedup mode every id
// also sets its token's bit in its rank's bitmap (setting it twice is harmless).
// `s_rank` maps expert -> rank (LDS) or is null for contiguous placement.
// PAD (received rows): negative ids are empty slots and only the first
// `tvalid` rows of the tile are counted; empty entries get the code kNoSlot.
template <bool DEDUP, bool PAD, int KMAX>
__device__ __forceinline__ void count_tile(const int (&raw)[KMAX], int64_t f0, int nf, int k,
                                           uint32_t kmul, int E, const int32_t* s_rank, int m,
                                           int tvalid, uint64_t* bits,
                                           uint32_t* __restrict__ lslot, int lane) {
  int e[KMAX], col[KMAX], tl[KMAX];
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    const int f = lane + kWave * r;
    e[r] = clampi(raw[r], 0, E - 1);
    tl[r] = kdiv(uint32_t(f), kmul, k);
    tl[r] = tl[r] < kTile ? tl[r] : kTile - 1;  // positions past the tile are never used
    col[r] = DEDUP ? (s_rank ? s_rank[e[r]] : e[r] / m) : e[r];
  }
  bool ok[KMAX];
#pragma unroll
  for (int r = 0; r < KMAX; ++r)
    ok[r] = lane + kWave * r < nf && (!PAD || (raw[r] >= 0 && tl[r] < tvalid));
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    if (ok[r]) {
      const unsigned long long bit = 1ull << tl[r];
      atomicOr(reinterpret_cast<unsigned long long*>(&bits[e[r]]), bit);
      if (DEDUP) atomicOr(reinterpret_cast<unsigned long long*>(&bits[E + col[r]]), bit);
    }
  }
  wave_lds_sync();
  uint32_t code[KMAX];
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    const uint64_t mb = bits[DEDUP ? E + col[r] : col[r]];
    const uint64_t below = tl[r] == 0 ? 0ull : (~0ull >> (kWave - tl[r]));
    code[r] = (uint32_t(col[r]) << 8) | uint32_t(__popcll(mb & below));
    if (PAD && !ok[r]) code[r] = kNoSlot;
  }
#pragma unroll
  for (int r = 0; r < KMAX; ++r)
    if (lane + kWave * r < nf) lslot[f0 + lane + kWave * r] = code[r];
}

// ----------------------------------------------------------- tile counts --

template <bool DEDUP, bool PAD, int KMAX>
__global__ void __launch_bounds__(kWave)
tile_counts_kernel(const int32_t* __restrict__ idx, int64_t T, int E, int k, int R,
                   const int32_t* __restrict__ place, int m, uint32_t kmul, int64_t Bp,
                   const int32_t* __restrict__ n_valid, uint8_t* __restrict__ tcnt,
                   uint32_t* __restrict__ lslot) {
  extern __shared__ uint64_t s_tdyn[];
  const int C = E + (DEDUP ? R : 0);
  uint64_t* bits = s_tdyn;                                        // [C]
  int32_t* s_rank = reinterpret_cast<int32_t*>(s_tdyn + C);      // [E] (dedup, explicit placement)
  const int lane = lane_id();
  const int64_t b = blockIdx.x;
  const int64_t f0 = b * kTile * k;
  const int64_t total = T * k;
  const int nf = int(total - f0 < int64_t(kTile) * k ? total - f0 : int64_t(kTile) * k);
  int raw[KMAX];
  load_tile_ids<KMAX>(raw, idx, f0, total, lane);
  int tvalid = kTile;  // rows of this tile that count (PAD: rows below *n_valid)
  if (PAD) {
    const int64_t nv = *n_valid;
    tvalid = int(nv - b * kTile < 0 ? 0 : (nv - b * kTile > kTile ? kTile : nv - b * kTile));
  }
  for (int c = lane; c < C; c += kWave) bits[c] = 0ull;
  const bool has_rank = DEDUP && place;
  if (has_rank)
    for (int e = lane; e < E; e += kWave) s_rank[e] = clampi(place[e], 0, R - 1);
  wave_lds_sync();
  count_tile<DEDUP, PAD, KMAX>(raw, f0, nf, k, kmul, E, has_rank ? s_rank : nullptr, m, tvalid,
                               bits, lslot, lane);
  for (int c = lane; c < C; c += kWave) tcnt[c * Bp + b] = uint8_t(__popcll(bits[c]));
}

// ------------------------------------------------------------------- scan --

constexpr int kScanThreads = 1024;
constexpr int kScanWaves = kScanThreads / kWave;
constexpr int kMaxCols = MOE_MAX_EXPERTS + MOE_MAX_RANKS;
constexpr int kMaxQ = 16;  // tile chunks per column
constexpr int kKeep = 8;   // 16-tile vectors a scan thread keeps in registers

// Sum of the 16 bytes of v (v_sad_u8 against zero adds four bytes at a time).
__device__ __forceinline__ int byte_sum(const u32x4& v) {
  uint32_t s = __builtin_amdgcn_sad_u8(v.x, 0u, 0u);
  s = __builtin_amdgcn_sad_u8(v.y, 0u, s);
  s = __builtin_amdgcn_sad_u8(v.z, 0u, s);
  s = __builtin_amdgcn_sad_u8(v.w, 0u, s);
  return int(s);
}

// Keeps the first n bytes of v and zeroes the rest (n <= 0: all zero).  The
// padding tiles B..Bp-1 of a column are never written by tile_counts.
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

// Writes the running first row of 16 consecutive tiles of one position column.
__device__ __forceinline__ void put_bases(const u32x4& v, int32_t& run, int32_t* dst) {
  int32_t o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    o[i] = run;
    run += int32_t((v[i / 4] >> (8 * (i % 4))) & 255u);
  }
  u32x4* d4 = reinterpret_cast<u32x4*>(dst);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    d4[i] = u32x4{uint32_t(o[4 * i]), uint32_t(o[4 * i + 1]), uint32_t(o[4 * i + 2]),
                  uint32_t(o[4 * i + 3])};
}

// One workgroup.  Each column's Bp/16 tile vectors are split into Q chunks,
// one (column, chunk) unit per thread: chunk sums, then per chunk the sum of
// the column's earlier chunks and the column total; experts are ordered by
// (rank, id) with a counting sort and one block-wide scan; then every unit of
// a position column writes the absolute first row of each of its tiles.
// KEEP: each thread owns at most one unit of at most kKeep vectors and keeps
// them in registers between the two passes; otherwise units loop and the
// second pass loads its vectors again (large inputs only).
template <bool DEDUP, bool KEEP>
__global__ void __launch_bounds__(kScanThreads)
plan_scan_kernel(const uint8_t* __restrict__ tcnt, int B, int Bp, int Q, int E, int R,
                 const int32_t* __restrict__ place, int m, int32_t* __restrict__ expert_counts,
                 int32_t* __restrict__ rank_counts, int32_t* __restrict__ rank_offsets,
                 int32_t* __restrict__ expert_offsets, int32_t* __restrict__ header,
                 int32_t* __restrict__ base) {
  __shared__ int32_t s_part[kMaxCols];  // [c][q] chunk sums
  __shared__ int32_t s_pre[kMaxCols];   // [c][q] sums of the column's earlier chunks
  __shared__ int32_t s_tot[kMaxCols];   // column totals
  __shared__ int32_t s_colbase[MOE_MAX_EXPERTS];
  __shared__ int32_t s_sorted[MOE_MAX_EXPERTS];
  __shared__ uint64_t s_rmask[MOE_MAX_RANKS][MOE_MAX_EXPERTS / kWave];
  __shared__ int32_t s_rcnt[MOE_MAX_RANKS];
  __shared__ int32_t s_rstart[MOE_MAX_RANKS + 1];
  __shared__ int32_t s_ro[MOE_MAX_RANKS + 1];
  __shared__ int32_t s_wsum[kScanWaves];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid / kWave;
  const int C = E + (DEDUP ? R : 0);
  const int cbase = DEDUP ? E : 0;  // first position column among the counted ones
  const int nvec = Bp / 16;         // 16-tile vectors per column
  const int units = C * Q;
  const int EW = (E + kWave - 1) / kWave;  // 64-expert words
  const bool sorted_by_id = DEDUP || place == nullptr;  // (rank, id) order == id order
  const u32x4* g4 = reinterpret_cast<const u32x4*>(tcnt);

  // 1. chunk sums (the loads go out first, before anything else)
  u32x4 keep[KEEP ? kKeep : 1];
  int kv0 = 0, kv1 = 0;
  if (KEEP) {
    if (tid < units) {
      const int c = tid / Q, q = tid - (tid / Q) * Q;
      kv0 = int(int64_t(nvec) * q / Q);
      kv1 = int(int64_t(nvec) * (q + 1) / Q);
#pragma unroll
      for (int i = 0; i < kKeep; ++i) {
        const int vi = kv0 + i < kv1 ? kv0 + i : kv1 - 1;  // every unit has a vector
        keep[i] = g4[size_t(c) * nvec + vi];
      }
    }
  }
  int my_rank = 0;  // rank of the expert this thread owns (place is wave-uniform)
  if (tid < E) my_rank = place ? clampi(place[tid], 0, R - 1) : tid / m;
  if (tid < MOE_MAX_RANKS) s_rcnt[tid] = 0;
  for (int i = tid; i < MOE_MAX_RANKS * (MOE_MAX_EXPERTS / kWave); i += kScanThreads)
    (&s_rmask[0][0])[i] = 0ull;
  if (KEEP) {
    if (tid < units) {
      int sum = 0;
#pragma unroll
      for (int i = 0; i < kKeep; ++i) {
        keep[i] = keep_bytes(keep[i], kv0 + i < kv1 ? B - 16 * (kv0 + i) : 0);
        sum += byte_sum(keep[i]);
      }
      s_part[tid] = sum;
    }
  } else {
    for (int u = tid; u < units; u += kScanThreads) {
      const int c = u / Q, q = u - (u / Q) * Q;
      const int v0 = int(int64_t(nvec) * q / Q), v1 = int(int64_t(nvec) * (q + 1) / Q);
      int sum = 0;
      for (int vi = v0; vi < v1; ++vi)
        sum += byte_sum(keep_bytes(g4[size_t(c) * nvec + vi], B - 16 * vi));
      s_part[u] = sum;
    }
  }
  __syncthreads();
  if (!sorted_by_id && tid < E) {
    atomicOr(reinterpret_cast<unsigned long long*>(&s_rmask[my_rank][tid / kWave]),
             1ull << (tid % kWave));
    atomicAdd(&s_rcnt[my_rank], 1);
  }

  // 2. chunk prefixes and column totals
  for (int u = tid; u < units; u += kScanThreads) {
    const int c = u / Q, q = u - (u / Q) * Q;
    const int32_t* part = s_part + c * Q;
    int32_t pre = 0;
#pragma unroll
    for (int qq = 0; qq < kMaxQ; ++qq) pre += qq < q ? part[qq < Q ? qq : 0] : 0;
    s_pre[u] = pre;
    if (q == Q - 1) s_tot[c] = pre + part[q];
  }
  __syncthreads();
  // start of each rank in the (rank, id) expert order
  if (!sorted_by_id && w == 0) {
    const int v = lane < R ? s_rcnt[lane] : 0;
    const int incl = wave_incl_scan(v);
    if (lane < R) s_rstart[lane] = incl - v;
  }
  __syncthreads();

  // 3. the expert order: expert e goes to slot `key` of the (rank, id) order
  int key = tid;
  if (!sorted_by_id && tid < E) {
    const uint64_t* mk = s_rmask[my_rank];
    const int wi = tid / kWave;
    int below = __popcll(mk[wi] & lanemask_lt());
#pragma unroll
    for (int q = 0; q < MOE_MAX_EXPERTS / kWave; ++q) below += q < wi ? __popcll(mk[q]) : 0;
    key = s_rstart[my_rank] + below;
  }
  if (!DEDUP && tid < E) s_sorted[key] = s_tot[tid];
  __syncthreads();

  // 4. exclusive scan in that order (experts, or ranks in dedup mode)
  const int nscan = DEDUP ? R : E;
  const int nsw = (nscan + kWave - 1) / kWave;
  int v = 0;
  if (tid < nscan) v = DEDUP ? s_tot[E + tid] : s_sorted[tid];
  int incl = 0;
  if (w < nsw) {
    incl = wave_incl_scan(v);
    if (lane == kWave - 1) s_wsum[w] = incl;
  }
  __syncthreads();
  int carry = 0;
#pragma unroll
  for (int q = 0; q < kScanWaves; ++q) carry += q < w ? s_wsum[q < EW ? q : 0] : 0;
  const int excl = carry + incl - v;
  if (tid < nscan) s_sorted[tid] = excl;  // scanned value of slot tid
  if (tid == 0) {
    int total = 0;
#pragma unroll
    for (int q = 0; q < kScanWaves; ++q) total += q < nsw ? s_wsum[q] : 0;
    s_ro[R] = total;
    header[0] = total;
  }
  __syncthreads();

  // 5. counts, offsets and column bases
  if (tid < E) expert_counts[tid] = s_tot[tid];
  if (!DEDUP) {
    if (tid < E) {
      const int off = s_sorted[key];
      s_colbase[tid] = off;
      if (expert_offsets) expert_offsets[tid] = off;
    }
    if (tid < R) {
      // the first expert of rank r in the (rank, id) order
      const int first = sorted_by_id ? tid * m : s_rstart[tid];
      s_ro[tid] = first < E ? s_sorted[first] : s_ro[R];
    }
  } else if (tid < R) {
    s_ro[tid] = s_sorted[tid];
    s_colbase[tid] = s_sorted[tid];
  }
  __syncthreads();
  if (tid < R) rank_counts[tid] = s_ro[tid + 1] - s_ro[tid];
  if (tid <= R) rank_offsets[tid] = s_ro[tid];

  // 6. absolute first row of every (position column, tile)
  if (KEEP) {
    if (tid < units && tid >= cbase * Q) {
      const int c = tid / Q;
      const int cp = c - cbase;
      int32_t run = s_colbase[cp] + s_pre[tid];
      int32_t* col = base + size_t(cp) * Bp;
#pragma unroll
      for (int i = 0; i < kKeep; ++i)
        if (kv0 + i < kv1) put_bases(keep[i], run, col + 16 * (kv0 + i));
    }
  } else {
    for (int u = cbase * Q + tid; u < units; u += kScanThreads) {
      const int c = u / Q, q = u - (u / Q) * Q;
      const int cp = c - cbase;
      const int v0 = int(int64_t(nvec) * q / Q), v1 = int(int64_t(nvec) * (q + 1) / Q);
      int32_t run = s_colbase[cp] + s_pre[u];
      int32_t* col = base + size_t(cp) * Bp;
      for (int vi = v0; vi < v1; ++vi)
        put_bases(keep_bytes(g4[size_t(c) * nvec + vi], B - 16 * vi), run, col + 16 * vi);
    }
  }
}

// Inclusive scan inside aligned segments of Q consecutive lanes (Q a power of
// two <= 16, so a segment never leaves its 16-lane DPP row).
__device__ __forceinline__ int segment_incl_scan(int v, int Q, int lane) {
  const int ls = lane & (Q - 1);
  int t = __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += ls >= 1 ? t : 0;
  t = __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);      // row_shr:2
  v += (Q > 2 && ls >= 2) ? t : 0;
  t = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);      // row_shr:4
  v += (Q > 4 && ls >= 4) ? t : 0;
  t = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);      // row_shr:8
  v += (Q > 8 && ls >= 8) ? t : 0;
  return v;
}

// The common cases in one pass with two barriers: plain mode with contiguous
// placement (the scan order is the expert id order) and dedup mode (the scan
// order is the rank order).  One (column, chunk) unit per thread, Q chunks per
// column (a power of two) on consecutive lanes, each of at most KV vectors; the
// workgroup has just enough waves for the units.
// A unit's byte sum is scanned inside its column's lane segment (DPP); the
// segment's last lane carries the column total into one block-wide scan over
// all units, whose exclusive value at any unit of a column is the column's
// first row; each unit then writes its tiles' bases from the vectors it kept.
template <bool DEDUP, int KV>
__global__ void __launch_bounds__(kScanThreads)
plan_scan_fast_kernel(const uint8_t* __restrict__ tcnt, int B, int Bp, int Q, int E, int R, int m,
                      int32_t* __restrict__ expert_counts, int32_t* __restrict__ rank_counts,
                      int32_t* __restrict__ rank_offsets, int32_t* __restrict__ expert_offsets,
                      int32_t* __restrict__ header, int32_t* __restrict__ base) {
  __shared__ int32_t s_wsum[kScanWaves];
  __shared__ int32_t s_ro[MOE_MAX_RANKS + 1];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid / kWave;
  const int nwaves = blockDim.x / kWave;
  const int C = E + (DEDUP ? R : 0);
  const int cbase = DEDUP ? E : 0;
  const int nvec = Bp / 16;
  const int units = C * Q;
  const bool active = tid < units;
  const int c = tid / Q, q = tid & (Q - 1);
  const int v0 = int(int64_t(nvec) * q / Q), v1 = int(int64_t(nvec) * (q + 1) / Q);
  const u32x4* g4 = reinterpret_cast<const u32x4*>(tcnt);
  u32x4 keep[KV];
#pragma unroll
  for (int i = 0; i < KV; ++i) {
    const int vi = v0 + i < v1 ? v0 + i : v1 - 1;  // every unit has a vector
    keep[i] = g4[size_t(active ? c : 0) * nvec + vi];
  }
  int part = 0;
#pragma unroll
  for (int i = 0; i < KV; ++i) {
    keep[i] = keep_bytes(keep[i], v0 + i < v1 ? B - 16 * (v0 + i) : 0);
    part += byte_sum(keep[i]);
  }
  part = active ? part : 0;
  const int incl_c = segment_incl_scan(part, Q, lane);
  const int tot = __shfl(incl_c, (lane & ~(Q - 1)) + Q - 1, kWave);  // column total
  const int pre = incl_c - part;                                      // earlier chunks
  const bool pos = active && c >= cbase;
  const int v = (pos && q == Q - 1) ? tot : 0;
  const int incl = wave_incl_scan(v);
  if (lane == kWave - 1) s_wsum[w] = incl;
  __syncthreads();
  int carry = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kScanWaves; ++i) {
    const int x = i < nwaves ? s_wsum[i < nwaves ? i : 0] : 0;
    carry += i < w ? x : 0;
    total += x;
  }
  const int colbase = carry + incl - v;  // first row of this unit's column
  if (active && q == 0) {
    if (c < E) expert_counts[c] = tot;
    if (DEDUP && c >= E) {
      rank_counts[c - E] = tot;
      rank_offsets[c - E] = colbase;
    }
    if (!DEDUP) {
      if (expert_offsets) expert_offsets[c] = colbase;
      if (c % m == 0) s_ro[c / m] = colbase;
    }
  }
  if (tid == 0) {
    header[0] = total;
    rank_offsets[R] = total;
    if (!DEDUP) s_ro[R] = total;
  }
  if (pos) {
    int32_t run = colbase + pre;
    int32_t* col = base + size_t(c - cbase) * Bp;
#pragma unroll
    for (int i = 0; i < KV; ++i)
      if (v0 + i < v1) put_bases(keep[i], run, col + 16 * (v0 + i));
  }
  if (!DEDUP) {
    __syncthreads();
    if (tid < R) {
      rank_offsets[tid] = s_ro[tid];
      rank_counts[tid] = s_ro[tid + 1] - s_ro[tid];
    }
  }
}

template <bool PAD, int KMAX>
static hipError_t launch_counts_k(const int32_t* idx, int64_t T, int E, int k, int R,
                                  const int32_t* place, int dedup, const int32_t* n_valid,
                                  int32_t* expert_counts, int32_t* rank_counts,
                                  int32_t* rank_offsets, int32_t* expert_offsets,
                                  void* workspace, hipStream_t stream) {
  const PlanLayout pl = plan_layout(T, E, k, R, dedup);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* header = reinterpret_cast<int32_t*>(ws);
  int32_t* base = reinterpret_cast<int32_t*>(ws + pl.base_off);
  uint8_t* tcnt = ws + pl.tcnt_off;
  uint32_t* lslot = reinterpret_cast<uint32_t*>(ws + pl.lslot_off);
  const int m = E / R;
  if (T > 0) {
    const size_t lds = size_t(pl.cols) * sizeof(uint64_t) + size_t(E) * sizeof(int32_t);
    const uint32_t kmul = kdiv_mul(k);
    if (dedup)
      hipLaunchKernelGGL((tile_counts_kernel<true, false, KMAX>), dim3(unsigned(pl.tiles)),
                         dim3(kWave), lds, stream, idx, T, E, k, R, place, m, kmul, pl.tiles_pad,
                         n_valid, tcnt, lslot);
    else
      hipLaunchKernelGGL((tile_counts_kernel<false, PAD, KMAX>), dim3(unsigned(pl.tiles)),
                         dim3(kWave), lds, stream, idx, T, E, k, R, place, m, kmul, pl.tiles_pad,
                         n_valid, tcnt, lslot);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int B = int(pl.tiles);
  const int Bp = int(pl.tiles_pad);
  const int nvec = Bp / 16;
  // fast path: chunks per column a power of two, one unit per thread, at most
  // kKeep vectors per unit; plain mode only with contiguous placement
  if (nvec > 0 && (dedup || place == nullptr)) {
    int Qf = kMaxQ;
    while (Qf > 1 && (pl.cols * Qf > kScanThreads || Qf > nvec)) Qf >>= 1;
    const int kv = (nvec + Qf - 1) / Qf;
    if (pl.cols * Qf <= kScanThreads && kv <= kKeep) {
      const int threads = (pl.cols * Qf + kWave - 1) / kWave * kWave;
#define MOE_FAST_SCAN(D, KV)                                                                     \
  hipLaunchKernelGGL((plan_scan_fast_kernel<D, KV>), dim3(1), dim3(threads), 0, stream, tcnt, B, \
                     Bp, Qf, E, R, m, expert_counts, rank_counts, rank_offsets, expert_offsets,   \
                     header, base)
#define MOE_FAST_SCAN_KV(D)       \
  if (kv <= 1) MOE_FAST_SCAN(D, 1); \
  else if (kv <= 2) MOE_FAST_SCAN(D, 2); \
  else if (kv <= 4) MOE_FAST_SCAN(D, 4); \
  else MOE_FAST_SCAN(D, 8);
      if (dedup) {
        MOE_FAST_SCAN_KV(true)
      } else {
        MOE_FAST_SCAN_KV(false)
      }
#undef MOE_FAST_SCAN_KV
#undef MOE_FAST_SCAN
      return hipGetLastError();
    }
  }
  int Q = kScanThreads / pl.cols;
  Q = Q < 1 ? 1 : (Q > kMaxQ ? kMaxQ : Q);
  Q = Q < nvec ? Q : (nvec > 0 ? nvec : 1);
  // one unit per thread, each of at most kKeep vectors
  const bool keep = nvec > 0 && pl.cols * Q <= kScanThreads && (nvec + Q - 1) / Q <= kKeep;
#define MOE_SCAN_LAUNCH(D, K)                                                                   \
  hipLaunchKernelGGL((plan_scan_kernel<D, K>), dim3(1), dim3(kScanThreads), 0, stream, tcnt, B,  \
                     Bp, Q, E, R, place, m, expert_counts, rank_counts, rank_offsets,            \
                     expert_offsets, header, base)
  if (dedup) {
    if (keep) MOE_SCAN_LAUNCH(true, true);
    else MOE_SCAN_LAUNCH(true, false);
  } else {
    if (keep) MOE_SCAN_LAUNCH(false, true);
    else MOE_SCAN_LAUNCH(false, false);
  }
#undef MOE_SCAN_LAUNCH
  return hipGetLastError();
}

hipError_t launch_send_counts(const int32_t* idx, int64_t T, int E, int k, int R,
                              const int32_t* place, int dedup, int32_t* expert_counts,
                              int32_t* rank_counts, int32_t* rank_offsets,
                              int32_t* expert_offsets, void* workspace, hipStream_t stream) {
  if (k <= 2)
    return launch_counts_k<false, 2>(idx, T, E, k, R, place, dedup, nullptr, expert_counts,
                                     rank_counts, rank_offsets, expert_offsets, workspace,
                                     stream);
  if (k <= 4)
    return launch_counts_k<false, 4>(idx, T, E, k, R, place, dedup, nullptr, expert_counts,
                                     rank_counts, rank_offsets, expert_offsets, workspace,
                                     stream);
  if (k <= 8)
    return launch_counts_k<false, 8>(idx, T, E, k, R, place, dedup, nullptr, expert_counts,
                                     rank_counts, rank_offsets, expert_offsets, workspace,
                                     stream);
  return launch_counts_k<false, 16>(idx, T, E, k, R, place, dedup, nullptr, expert_counts,
                                    rank_counts, rank_offsets, expert_offsets, workspace, stream);
}

// Receive side: the plan of the per-expert expansion of `cap` received rows, of
// which the first *n_rows count; negative ids are empty slots.  Same plan as
// the plain dispatch (rows play the part of tokens).
hipError_t launch_expand_counts(const int32_t* row_experts, int64_t cap, int E, int k, int R,
                                const int32_t* place, const int32_t* n_rows,
                                int32_t* expert_counts, int32_t* rank_counts,
                                int32_t* rank_offsets, int32_t* expert_offsets, void* workspace,
                                hipStream_t stream) {
  if (k <= 2)
    return launch_counts_k<true, 2>(row_experts, cap, E, k, R, place, 0, n_rows, expert_counts,
                                    rank_counts, rank_offsets, expert_offsets, workspace,
                                    stream);
  if (k <= 4)
    return launch_counts_k<true, 4>(row_experts, cap, E, k, R, place, 0, n_rows, expert_counts,
                                    rank_counts, rank_offsets, expert_offsets, workspace,
                                    stream);
  if (k <= 8)
    return launch_counts_k<true, 8>(row_experts, cap, E, k, R, place, 0, n_rows, expert_counts,
                                    rank_counts, rank_offsets, expert_offsets, workspace,
                                    stream);
  return launch_counts_k<true, 16>(row_experts, cap, E, k, R, place, 0, n_rows, expert_counts,
                                   rank_counts, rank_offsets, expert_offsets, workspace, stream);
}

}  // namespace moe
