// The column order and block-wide scan of a dispatch plan, shared by the scan
// kernels (counts.hip) and the dispatch kernels that scan a small plan
// themselves (dispatch.hip): from the column totals, every position column's
// first row in the send buffer, and optionally the counts and offsets.
#pragma once

#include "common.hpp"
#include "moe_route.h"

namespace moe {

constexpr int kScanThreads = 1024;
constexpr int kScanWaves = kScanThreads / kWave;
constexpr int kMaxCols = MOE_MAX_EXPERTS + MOE_MAX_RANKS;

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

// LDS of the column-order scan (order_columns), declared by its caller.
template <bool RANKED>
struct OrderLds {
  int32_t scan[MOE_MAX_EXPERTS];  // exclusive scan by scan slot (RANKED)
  int32_t wsum[kScanWaves];
  uint64_t rmask[RANKED ? MOE_MAX_RANKS : 1][MOE_MAX_EXPERTS / kWave];
  int32_t rcnt[MOE_MAX_RANKS];
  int32_t rstart[MOE_MAX_RANKS];
};

// Clears the rank bitmaps and counts of L (RANKED); every thread calls it,
// and a barrier must follow before order_columns.
template <bool RANKED>
__device__ __forceinline__ void order_init(OrderLds<RANKED>& L) {
  if (!RANKED) return;
  const int tid = threadIdx.x;
  if (tid < MOE_MAX_RANKS) L.rcnt[tid] = 0;
  for (int i = tid; i < MOE_MAX_RANKS * (MOE_MAX_EXPERTS / kWave); i += blockDim.x)
    (&L.rmask[0][0])[i] = 0ull;
}

// The position columns in send-buffer order - expert id (plain, contiguous
// placement), rank (dedup), or (rank, id) for plain dispatch with an explicit
// placement (RANKED: a counting sort with rank bitmasks) - and one
// block-wide exclusive scan (DPP wave scans) of their totals s_tot give each
// position column's first row, s_colbase[0 .. CP).  With `outputs`, also the
// counts, the offsets and the header.  Every thread of the workgroup calls it
// after s_tot is complete and order_init's barrier; the workgroup has at least
// max(CP, R) threads and, RANKED, at least E (my_rank: the rank of expert tid).
// Returns the total number of rows.
template <bool DEDUP, bool RANKED>
__device__ int order_columns(const int32_t* s_tot, int32_t* s_colbase, OrderLds<RANKED>& L,
                             int E, int R, int m, int my_rank, bool outputs,
                             int32_t* __restrict__ expert_counts,
                             int32_t* __restrict__ rank_counts,
                             int32_t* __restrict__ rank_offsets,
                             int32_t* __restrict__ expert_offsets,
                             int32_t* __restrict__ header) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid / kWave;
  const int nwaves = blockDim.x / kWave;
  const int cbase = DEDUP ? E : 0;  // first position column among the counted ones
  const int CP = DEDUP ? R : E;     // position columns = scan slots
  int key = tid;  // scan slot of expert tid (RANKED), else slot tid = column cbase + tid
  if (RANKED) {
    if (tid < E) {
      atomicOr(reinterpret_cast<unsigned long long*>(&L.rmask[my_rank][tid / kWave]),
               1ull << (tid % kWave));
      atomicAdd(&L.rcnt[my_rank], 1);
    }
    __syncthreads();
    if (w == 0) {
      const int v = lane < R ? L.rcnt[lane] : 0;
      const int incl = wave_incl_scan(v);
      if (lane < R) L.rstart[lane] = incl - v;
    }
    __syncthreads();
    if (tid < E) {
      const uint64_t* mk = L.rmask[my_rank];
      const int wi = tid / kWave;
      int below = __popcll(mk[wi] & lanemask_lt());
#pragma unroll
      for (int qq = 0; qq < MOE_MAX_EXPERTS / kWave; ++qq) below += qq < wi ? __popcll(mk[qq]) : 0;
      key = L.rstart[my_rank] + below;
      L.scan[key] = s_tot[tid];
    }
    __syncthreads();
  }
  const int sv = tid < CP ? (RANKED ? L.scan[tid] : s_tot[cbase + tid]) : 0;
  const int incl = wave_incl_scan(sv);
  if (lane == kWave - 1) L.wsum[w] = incl;
  __syncthreads();
  int carry = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kScanWaves; ++i) {
    const int x = i < nwaves ? L.wsum[i < nwaves ? i : 0] : 0;
    carry += i < w ? x : 0;
    total += x;
  }
  const int excl = carry + incl - sv;  // first row of scan slot tid
  if (RANKED) {
    __syncthreads();  // every L.scan read above is done
    if (tid < CP) L.scan[tid] = excl;
    __syncthreads();
    if (tid < E) s_colbase[tid] = L.scan[key];
  } else if (tid < CP) {
    s_colbase[tid] = excl;
  }
  __syncthreads();
  if (outputs) {
    if (tid < E) expert_counts[tid] = s_tot[tid];
    if (!DEDUP && expert_offsets && tid < E) expert_offsets[tid] = s_colbase[tid];
    if (tid < R) {
      int start, next;
      if (DEDUP) {
        start = s_colbase[tid];
        next = start + s_tot[E + tid];
      } else if (RANKED) {
        const int s0 = L.rstart[tid], s1 = tid + 1 < R ? L.rstart[tid + 1] : E;
        start = s0 < E ? L.scan[s0] : total;
        next = s1 < E ? L.scan[s1] : total;
      } else {
        start = s_colbase[tid * m];
        next = tid + 1 < R ? s_colbase[(tid + 1) * m] : total;
      }
      rank_offsets[tid] = start;
      rank_counts[tid] = next - start;
    }
    if (tid == 0) {
      rank_offsets[R] = total;
      header[0] = total;
    }
  }
  return total;
}

}  // namespace moe
