// A4a / A4b - dispatch permute into a rank-contiguous send buffer.
//
// Source: "Expert Coupling in MoE Pretraining" (summary), "Method 1: Correlated
// Expert Placement + Deduplicating Dispatcher": the conventional dispatcher
// sends one copy of a token's hidden state per (token, expert); the
// deduplicating one sends one row per distinct (token, destination rank) with
// the ids and routing probabilities of the rank's selected experts as
// metadata.  "DODOCO" dataset card, "Reading the counts": a token routed to
// several experts on one rank is counted (and sent) once per expert by the
// conventional dispatcher.
//
// Design: one wave per (token, row chunk).  Lanes j < k first resolve slot j's
// destination row from the plan (the tile's first row in the slot's column +
// the slot's rank inside the tile), then the wave
// reads its chunk of x[t] once into registers (16-byte loads, 1 KiB per wave
// instruction) and writes it to each destination row.  Every access is a full,
// contiguous row segment, so reads and writes are perfectly coalesced; nothing
// is re-read, so there is no cross-workgroup reuse for an XCD-aware order to
// exploit.  Chunk 0 of each token also writes the row metadata.
#include "common.hpp"

namespace moe {

// Loads are issued unconditionally from addresses clamped into the row, so a
// wave's loads go out back to back (a load under a lane-divergent branch is
// followed by a wait for it); only the stores are predicated.
template <int NV>
__device__ __forceinline__ void load_chunk(u32x4 (&v)[NV], const uint8_t* row, int64_t chunk0,
                                           int row_bytes, int lane) {
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int64_t off = chunk0 + int64_t(i * kWave + lane) * 16;
    off = off < row_bytes ? off : row_bytes - 16;
    v[i] = load16(row + off);
  }
}

// Keeps the row loads above it ahead of what follows.  Without it the compiler
// issues them after the position lookups (slot code, then the tile's counts),
// so each wave waits for three memory round trips in a row instead of
// overlapping the row with the lookups.  The row pointer `x` of the kernels is
// deliberately not __restrict__: loads through a restrict read-only pointer
// count as invariant, and the compiler moves those past the fence.
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

// First row of position column `col` in tile b: the scan's base of the tile's
// 16-tile group plus the counts of the group's earlier tiles (one 16-byte load
// of the column's tile counts).
__device__ __forceinline__ int tile_first_row(const int32_t* __restrict__ gbase,
                                              const uint8_t* __restrict__ tcnt, int64_t Bp,
                                              int64_t G, int tcol, int col, int64_t b) {
  const int g = int(gbase[col * G + (b >> 4)]);
  const u32x4 tv = load16(tcnt + tcol * Bp + (b & ~int64_t(15)));
  return g + byte_sum(keep_bytes(tv, int(b & 15)));
}

template <int NV, bool NT>
__device__ __forceinline__ void store_chunk(const u32x4 (&v)[NV], uint8_t* dst, int64_t chunk0,
                                            int row_bytes, int lane) {
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int64_t off = int64_t(i * kWave + lane) * 16;
    if (chunk0 + off < row_bytes) {
      if (NT)
        store16_nt(dst + off, v[i]);
      else
        store16(dst + off, v[i]);
    }
  }
}

// PAD: the receive-side expansion, where a "token" is a received row, slots
// with the code kNoSlot are empty, only rows below *n_valid are expanded, and
// no row is written at or past out_cap (such slots get slot_row = -1).
template <int NV, bool NT, bool PAD>
__global__ void __launch_bounds__(256)
dispatch_kernel(const uint8_t* x, const float* __restrict__ gate, int64_t T,
                int row_bytes, int k, int cpr, const int32_t* __restrict__ gbase,
                const uint8_t* __restrict__ tcnt, const uint32_t* __restrict__ lslot, int64_t Bp,
                int64_t G, uint8_t* __restrict__ send,
                int32_t* __restrict__ row_token, int32_t* __restrict__ row_expert,
                float* __restrict__ row_weight, int32_t* __restrict__ slot_row,
                const int32_t* __restrict__ n_valid, int64_t out_cap) {
  const int lane = lane_id();
  const int64_t wid = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;
  const int64_t t = wid / cpr;
  const int c = int(wid - t * cpr);
  if (t >= T) return;  // whole wave
  if (PAD && t >= *n_valid) {  // whole wave: a row past the received ones
    if (c == 0 && lane < k) slot_row[t * k + lane] = -1;
    return;
  }
  const int64_t chunk0 = int64_t(c) * (NV * kWave * 16);
  // lanes j < k own slot j; the other lanes load slot k-1's data and ignore it
  const int jl = lane < k ? lane : k - 1;
  const uint32_t code = lslot[t * k + jl];  // (expert << 8) | rank inside the tile
  const float g = gate[t * k + jl];
  u32x4 v[NV];
  load_chunk<NV>(v, x + t * row_bytes, chunk0, row_bytes, lane);
  issue_fence();
  const bool has = !PAD || code != kNoSlot;
  const int e = has ? int(code >> 8) : 0;
  const int pos = tile_first_row(gbase, tcnt, Bp, G, e, e, t / kTile) + int(code & 255u);
  const bool ok = has && (!PAD || pos < out_cap);
  const uint64_t okm = __ballot(lane < k && ok);
  for (int j = 0; j < k; ++j) {
    if (PAD && !((okm >> j) & 1ull)) continue;
    const int p = bcast(pos, j);
    store_chunk<NV, NT>(v, send + int64_t(p) * row_bytes + chunk0, chunk0, row_bytes, lane);
  }
  // metadata last: stores count against the same wait counter as loads, so
  // stores issued before the row stores would hold them up
  if (c == 0 && lane < k) {
    slot_row[t * k + lane] = ok ? pos : -1;
    if (ok) {
      row_token[pos] = int32_t(t);
      row_expert[pos] = e;
      row_weight[pos] = g;
    }
  }
}

template <int NV, bool NT>
__global__ void __launch_bounds__(256)
dispatch_dedup_kernel(const uint8_t* x, const int32_t* __restrict__ idx,
                      const float* __restrict__ gate, int64_t T, int row_bytes, int E, int k,
                      int cpr, const int32_t* __restrict__ gbase, const uint8_t* __restrict__ tcnt,
                      const uint32_t* __restrict__ lslot, int64_t Bp, int64_t G,
                      const int32_t* __restrict__ header, uint8_t* __restrict__ send,
                      int32_t* __restrict__ row_token, int32_t* __restrict__ row_experts,
                      float* __restrict__ row_gates, float* __restrict__ row_weight,
                      int32_t* __restrict__ slot_row, int32_t* __restrict__ n_rows) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_rows = header[0];
  const int lane = lane_id();
  const int64_t wid = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;
  const int64_t t = wid / cpr;
  const int c = int(wid - t * cpr);
  if (t >= T) return;  // whole wave
  const int64_t chunk0 = int64_t(c) * (NV * kWave * 16);
  const int jl = lane < k ? lane : k - 1;
  const int e = clampi(idx[t * k + jl], 0, E - 1);
  const uint32_t code = lslot[t * k + jl];  // (rank << 8) | rank inside the tile
  const float g = gate[t * k + jl];
  u32x4 v[NV];
  load_chunk<NV>(v, x + t * row_bytes, chunk0, row_bytes, lane);
  issue_fence();
  const int r_own = int(code >> 8);
  const int pos = tile_first_row(gbase, tcnt, Bp, G, E + r_own, r_own, t / kTile) +
                  int(code & 255u);
  const int r = lane < k ? r_own : -1;  // lanes >= k match no slot below
  // Per slot: is it the first slot of its rank (the row's leader)?  Its column
  // among the rank's experts (ascending id), the rank's slot count, and its
  // position in the token's ascending expert order.
  bool leader = lane < k;
  int col = 0, cnt = 0, sidx = 0;
  for (int i = 0; i < k; ++i) {
    const int ri = bcast(r, i), ei = bcast(e, i);
    if (ri == r) {
      ++cnt;
      if (ei < e) ++col;
      if (i < lane) leader = false;
    }
    if (ei < e) ++sidx;
  }
  const uint64_t lm = __ballot(leader);
  for (int j = 0; j < k; ++j) {
    if (!((lm >> j) & 1ull)) continue;
    const int p = bcast(pos, j);
    store_chunk<NV, NT>(v, send + int64_t(p) * row_bytes + chunk0, chunk0, row_bytes, lane);
  }
  // metadata after the row stores (see the plain kernel)
  if (c == 0) {
    if (lane < k) {
      slot_row[t * k + lane] = pos;
      row_experts[int64_t(pos) * k + col] = e;
      row_gates[int64_t(pos) * k + col] = g;
      if (leader) {
        row_token[pos] = int32_t(t);
        for (int cc = cnt; cc < k; ++cc) {
          row_experts[int64_t(pos) * k + cc] = -1;
          row_gates[int64_t(pos) * k + cc] = 0.0f;
        }
      }
    }
    // row weight: fp64 sum of the rank's gates in ascending expert order
    double wsum = 0.0;
    for (int s = 0; s < k; ++s) {
      const uint64_t sm = __ballot(lane < k && sidx == s);
      if (sm == 0ull) continue;  // only if topk_idx repeats an expert (precondition)
      const int src = __ffsll((unsigned long long)sm) - 1;
      const float gs = bcastf(g, src);
      const int rs = bcast(r, src);
      if (leader && rs == r) wsum += double(gs);
    }
    if (leader) row_weight[pos] = float(wsum);
  }
}

#ifndef MOE_DISPATCH_NT
#define MOE_DISPATCH_NT 0
#endif

// Vectors of 16 B per lane per wave: a 4 KiB chunk per wave for long rows.
static int dispatch_nv(int row_bytes) {
  const int vr = row_bytes / 16;
  if (vr >= 4 * kWave) return 4;
  if (vr >= 2 * kWave) return 2;
  return 1;
}

template <int NV>
static hipError_t launch_dispatch_nv(const void* x, const int32_t* idx, const float* gate,
                                     int64_t T, int row_bytes, int E, int k, int R,
                                     const void* workspace, int dedup,
                                     void* send, int32_t* row_token, int32_t* row_e,
                                     float* row_gates, float* row_weight, int32_t* slot_row,
                                     int32_t* n_rows, hipStream_t stream) {
  const PlanLayout pl = plan_layout(T, E, k, R, dedup);
  const uint8_t* ws = static_cast<const uint8_t*>(workspace);
  const int32_t* header = reinterpret_cast<const int32_t*>(ws);
  const int32_t* gbase = reinterpret_cast<const int32_t*>(ws + pl.base_off);
  const uint8_t* tcnt = ws + pl.tcnt_off;
  const uint32_t* lslot = reinterpret_cast<const uint32_t*>(ws + pl.lslot_off);
  const int chunk = NV * kWave * 16;
  const int cpr = (row_bytes + chunk - 1) / chunk;
  const int64_t waves = T * cpr;
  int64_t blocks = (waves + 3) / 4;
  if (blocks == 0) blocks = 1;  // dedup still reports n_rows
  constexpr bool NT = MOE_DISPATCH_NT != 0;
  if (!dedup) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL((dispatch_kernel<NV, NT, false>), dim3(unsigned(blocks)), dim3(256), 0,
                       stream, static_cast<const uint8_t*>(x), gate, T, row_bytes, k, cpr, gbase,
                       tcnt, lslot, pl.tiles_pad, pl.groups, static_cast<uint8_t*>(send),
                       row_token, row_e, row_weight, slot_row, nullptr, int64_t(0));
  } else {
    hipLaunchKernelGGL((dispatch_dedup_kernel<NV, NT>), dim3(unsigned(blocks)), dim3(256), 0,
                       stream, static_cast<const uint8_t*>(x), idx, gate, T, row_bytes, E, k, cpr,
                       gbase, tcnt, lslot, pl.tiles_pad, pl.groups, header,
                       static_cast<uint8_t*>(send), row_token, row_e, row_gates, row_weight,
                       slot_row, n_rows);
  }
  return hipGetLastError();
}

hipError_t launch_dispatch(const void* x, const int32_t* idx, const float* gate, int64_t T,
                           int row_bytes, int E, int k, int R, const void* workspace, int dedup,
                           void* send, int32_t* row_token,
                           int32_t* row_e, float* row_gates, float* row_weight,
                           int32_t* slot_row, int32_t* n_rows, hipStream_t stream) {
  switch (dispatch_nv(row_bytes)) {
    case 4:
      return launch_dispatch_nv<4>(x, idx, gate, T, row_bytes, E, k, R, workspace, dedup,
                                   send, row_token, row_e, row_gates, row_weight, slot_row,
                                   n_rows, stream);
    case 2:
      return launch_dispatch_nv<2>(x, idx, gate, T, row_bytes, E, k, R, workspace, dedup,
                                   send, row_token, row_e, row_gates, row_weight, slot_row,
                                   n_rows, stream);
    default:
      return launch_dispatch_nv<1>(x, idx, gate, T, row_bytes, E, k, R, workspace, dedup,
                                   send, row_token, row_e, row_gates, row_weight, slot_row,
                                   n_rows, stream);
  }
}


template <int NV>
static hipError_t launch_expand_nv(const void* rows, const float* row_gates,
                                   const int32_t* n_rows, int64_t cap, int row_bytes, int E,
                                   int k, int R, const void* workspace, void* expanded,
                                   int64_t out_cap, int32_t* exp_row, int32_t* exp_expert,
                                   float* exp_gate, int32_t* row_slot, hipStream_t stream) {
  const PlanLayout pl = plan_layout(cap, E, k, R, 0);
  const uint8_t* ws = static_cast<const uint8_t*>(workspace);
  const int32_t* gbase = reinterpret_cast<const int32_t*>(ws + pl.base_off);
  const uint8_t* tcnt = ws + pl.tcnt_off;
  const uint32_t* lslot = reinterpret_cast<const uint32_t*>(ws + pl.lslot_off);
  const int chunk = NV * kWave * 16;
  const int cpr = (row_bytes + chunk - 1) / chunk;
  const int64_t blocks = (cap * cpr + 3) / 4;
  constexpr bool NT = MOE_DISPATCH_NT != 0;
  hipLaunchKernelGGL((dispatch_kernel<NV, NT, true>), dim3(unsigned(blocks)), dim3(256), 0,
                     stream, static_cast<const uint8_t*>(rows), row_gates, cap, row_bytes, k, cpr,
                     gbase, tcnt, lslot, pl.tiles_pad, pl.groups,
                     static_cast<uint8_t*>(expanded), exp_row, exp_expert, exp_gate, row_slot,
                     n_rows, out_cap);
  return hipGetLastError();
}

hipError_t launch_expand(const void* rows, const float* row_gates, const int32_t* n_rows,
                         int64_t cap, int row_bytes, int E, int k, int R, const void* workspace,
                         void* expanded, int64_t out_cap, int32_t* exp_row, int32_t* exp_expert,
                         float* exp_gate, int32_t* row_slot, hipStream_t stream) {
  if (cap == 0) return hipSuccess;
  switch (dispatch_nv(row_bytes)) {
    case 4:
      return launch_expand_nv<4>(rows, row_gates, n_rows, cap, row_bytes, E, k, R, workspace,
                                 expanded, out_cap, exp_row, exp_expert, exp_gate, row_slot,
                                 stream);
    case 2:
      return launch_expand_nv<2>(rows, row_gates, n_rows, cap, row_bytes, E, k, R, workspace,
                                 expanded, out_cap, exp_row, exp_expert, exp_gate, row_slot,
                                 stream);
    default:
      return launch_expand_nv<1>(rows, row_gates, n_rows, cap, row_bytes, E, k, R, workspace,
                                 expanded, out_cap, exp_row, exp_expert, exp_gate, row_slot,
                                 stream);
  }
}

}  // namespace moe
