// The combine's per-wave routine - the weighted sum of one token's rows for
// one output chunk - and its helpers, shared by the combine kernel
// (combine.hip) and the combine that also routes the next batch
// (combine_route.hip).  The method and the design are described in
// combine.hip.
#pragma once

#include "common.hpp"

#ifndef MOE_COMBINE_NT
#define MOE_COMBINE_NT 1
#endif
// Input vectors in flight per lane (KMAX rows x NV vectors) at most.
#ifndef MOE_COMBINE_VECS
#define MOE_COMBINE_VECS 24
#endif

namespace moe {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 f = {lo, hi};
  const bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

// One input vector per lane holds 8 values: 16 bytes of bf16, or 8 bytes of
// fp8 (IN8), so that its 8 bf16 outputs are always one 16-byte store and a
// wave instruction writes 1 KiB of contiguous output.
constexpr int kVals = 8;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <bool IN8>
struct InVec {
  typedef u32x4 type;
  static constexpr int kBytes = 16;
};
template <>
struct InVec<true> {
  typedef u32x2 type;
  static constexpr int kBytes = 8;
};

template <bool IN8, bool NT>
__device__ __forceinline__ typename InVec<IN8>::type load_in(const uint8_t* p) {
  typedef typename InVec<IN8>::type V;
  const V* q = reinterpret_cast<const V*>(p);
  return NT ? __builtin_nontemporal_load(q) : *q;
}

template <bool IN8>
__device__ __forceinline__ void decode(const typename InVec<IN8>::type& v, float (&f)[kVals]) {
#pragma unroll
  for (int h = 0; h < InVec<IN8>::kBytes / 4; ++h) {
    if constexpr (IN8) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(v[h]), false);  // bytes 0, 1
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(v[h]), true);   // bytes 2, 3
      f[4 * h] = lo.x;
      f[4 * h + 1] = lo.y;
      f[4 * h + 2] = hi.x;
      f[4 * h + 3] = hi.y;
    } else {
      f[2 * h] = __uint_as_float(v[h] << 16);
      f[2 * h + 1] = __uint_as_float(v[h] & 0xFFFF0000u);
    }
  }
}

// bf16 output of the kVals values of one input vector: 16 bytes at dst.
// NTS: nontemporal stores.
template <bool NTS>
__device__ __forceinline__ void store_out(uint8_t* dst, const float (&a)[kVals]) {
  u32x4 o;
#pragma unroll
  for (int h = 0; h < 4; ++h) o[h] = pack_bf16x2(a[2 * h], a[2 * h + 1]);
  if (NTS)
    store16_nt(dst, o);
  else
    store16(dst, o);
}

// The weighted sum of a token's rows for one chunk: NQ >= nrows rows are
// loaded (all loads before any arithmetic; rows past nrows repeat the first
// one and are not added), accumulated in fp32 from -0.0 in ascending row
// order, and stored as bf16.  `ord` is the lane's rank among the token's
// distinct rows (lanes without a row hold kNoOrder).  Offsets are in input
// bytes; output offsets are twice that for fp8 input.
template <int NQ, int NV, bool IN8, bool NTS>
__device__ __forceinline__ void sum_rows(const uint8_t* __restrict__ rows, int row_bytes,
                                         int64_t chunk0, int ord, int j0, int nrows, int rr,
                                         float wr, int lane, uint8_t* __restrict__ dst) {
  constexpr int OS = IN8 ? 2 : 1;  // output bytes per input byte
  constexpr int IB = InVec<IN8>::kBytes;
  typename InVec<IN8>::type y[NQ][NV];
  int jq[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    // the lane holding the q-th smallest row (q = 0: j0)
    const int j = (q > 0 && q < nrows) ? __ffsll((unsigned long long)__ballot(ord == q)) - 1 : j0;
    jq[q] = j;
    const int p = bcast(rr, j);
    const uint8_t* src = rows + int64_t(p) * row_bytes;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int64_t off = chunk0 + int64_t(i * kWave + lane) * IB;
      off = off < row_bytes ? off : row_bytes - IB;
      y[q][i] = load_in<IN8, MOE_COMBINE_NT != 0>(src + off);
    }
  }
  // the weights are broadcast only once every row load is out: reading the
  // weight register waits for its load, which would hold back the row loads
  // issued after it
  __builtin_amdgcn_sched_barrier(0);
  float wq[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) wq[q] = bcastf(wr, jq[q]);
  float acc[NV][kVals];
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int h = 0; h < kVals; ++h) acc[i][h] = -0.0f;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    if (q < nrows) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        float f[kVals];
        decode<IN8>(y[q][i], f);
#pragma unroll
        for (int h = 0; h < kVals; ++h) acc[i][h] = __builtin_fmaf(wq[q], f[h], acc[i][h]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int64_t off = chunk0 + int64_t(i * kWave + lane) * IB;
    if (off < row_bytes) store_out<NTS>(dst + OS * off, acc[i]);
  }
}

// Whether an earlier lane of the 16-lane DPP row holds the same value: lane j
// compares its value with lanes j-1 .. j-(KMAX-1), moved in with row_shr
// (lanes shifted in from before the row read a value no row index takes).
// Slots sit in lanes 0 .. k-1 <= KMAX-1 of row 0, so this finds a slot whose
// row an earlier slot already names, without a readlane per slot.
template <int S>
__device__ __forceinline__ int row_shr(int v) {
  return __builtin_amdgcn_update_dpp(int(0x80000000u), v, 0x110 + S, 0xF, 0xF, false);
}
template <int KMAX, int S = 1>
__device__ __forceinline__ bool repeats_earlier(int v) {
  if constexpr (S >= KMAX || S > 15) {
    return false;
  } else {
    return (row_shr<S>(v) == v) | repeats_earlier<KMAX, S + 1>(v);
  }
}

// Rank of lane j's key among the keys of lanes 0 .. KMAX-1 of its DPP row:
// the number of them that are smaller, counted over the lanes S below
// (row_shr) and S above (row_shl) for S = 1 .. KMAX-1.  Lanes shifted in from
// outside the row read INT_MAX, which is never smaller.  Keys are distinct
// except INT_MAX (lanes without a row), so the used lanes get ranks 0, 1, ...
// in ascending key order.
constexpr int kNoOrder = 64;
template <int S>
__device__ __forceinline__ int row_shr_max(int v) {
  return __builtin_amdgcn_update_dpp(0x7FFFFFFF, v, 0x110 + S, 0xF, 0xF, false);
}
template <int S>
__device__ __forceinline__ int row_shl_max(int v) {
  return __builtin_amdgcn_update_dpp(0x7FFFFFFF, v, 0x100 + S, 0xF, 0xF, false);
}
template <int KMAX, int S = 1>
__device__ __forceinline__ int rank_in_row(int v) {
  if constexpr (S >= KMAX || S > 15) {
    return 0;
  } else {
    return int(row_shr_max<S>(v) < v) + int(row_shl_max<S>(v) < v) + rank_in_row<KMAX, S + 1>(v);
  }
}

// Vectors per lane of one row chunk (NV): at most 4, and at most
// MOE_COMBINE_VECS / KMAX, so that KMAX x NV input vectors are in flight per
// lane; then as many as the row fills (a chunk is NV x 64 lanes x one vector).
template <int KMAX>
constexpr int combine_nv_max() {
  constexpr int q = MOE_COMBINE_VECS / KMAX;
  return q >= 4 ? 4 : (q > 0 ? q : 1);
}
template <int KMAX, bool IN8>
inline int combine_nv(int row_bytes) {
  constexpr int nvmax = combine_nv_max<KMAX>();
  const int vr = row_bytes / InVec<IN8>::kBytes;
  if (nvmax >= 4 && vr >= 4 * kWave) return 4;
  if (nvmax >= 2 && vr >= 2 * kWave) return 2;
  return 1;
}

// The calling wave's unit wid: chunk wid % cpr of output token wid / cpr.
template <int NV, int KMAX, bool IN8, bool NTS>
__device__ __forceinline__ void combine_unit(const uint8_t* __restrict__ rows,
                                             const float* __restrict__ w,
                                             const int32_t* __restrict__ slot_row, int64_t T,
                                             int row_bytes, int k, int cpr,
                                             const int32_t* __restrict__ n_valid,
                                             uint8_t* __restrict__ out, int64_t wid) {
  constexpr int OS = IN8 ? 2 : 1;
  const int lane = lane_id();
  const int64_t t = wid / cpr;
  const int c = int(wid - t * cpr);
  if (t >= T) return;  // whole wave
  if (n_valid && t >= *n_valid) return;  // whole wave: only the first *n_valid outputs
  constexpr int IB = InVec<IN8>::kBytes;
  const int64_t chunk0 = int64_t(c) * (NV * kWave * IB);
  // All loads are unconditional from clamped, in-bounds addresses (a load under
  // a branch is followed by a wait for it); only arithmetic and stores are
  // predicated.
  const int jl = lane < k ? lane : k - 1;
  const int r_raw = slot_row[t * k + jl];
  const int r = lane < k ? r_raw : -1;
  const bool use = (r >= 0) & !repeats_earlier<KMAX>(r);
  const uint64_t um = __ballot(use);
  const int nrows = __popcll(um);
  // rank of this lane's row among the token's distinct rows: rows are added in
  // ascending row index
  const int key = use ? r : 0x7FFFFFFF;  // every lane takes part in the DPP moves
  const int rk = rank_in_row<KMAX>(key);
  const int ord = use ? rk : kNoOrder;
  uint8_t* dst = out + t * int64_t(row_bytes) * OS;
  if (nrows == 0) {  // no row serves this token: the empty sum, -0.0
    const u32x4 nz = {0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int64_t off = chunk0 + int64_t(i * kWave + lane) * IB;
      if (off < row_bytes) store16(dst + OS * off, nz);
    }
    return;
  }
  const int j0 = __ffsll((unsigned long long)__ballot(ord == 0)) - 1;  // the smallest row
  const int rr = use ? r : bcast(r, j0);  // every lane names a valid row
  const float wr = w ? w[rr] : 1.0f;
  // as few row loads as the token needs (nrows is wave-uniform): a token served
  // by one or two rows - most received rows in the reduction - does not load
  // KMAX rows
  if constexpr (KMAX >= 1) {
    if (nrows <= 1)
      return sum_rows<1, NV, IN8, NTS>(rows, row_bytes, chunk0, ord, j0, nrows, rr, wr, lane, dst);
  }
  if constexpr (KMAX >= 2) {
    if (nrows <= 2)
      return sum_rows<2, NV, IN8, NTS>(rows, row_bytes, chunk0, ord, j0, nrows, rr, wr, lane, dst);
  }
  if constexpr (KMAX > 4) {
    if (nrows <= 4)
      return sum_rows<4, NV, IN8, NTS>(rows, row_bytes, chunk0, ord, j0, nrows, rr, wr, lane, dst);
  }
  sum_rows<KMAX, NV, IN8, NTS>(rows, row_bytes, chunk0, ord, j0, nrows, rr, wr, lane, dst);
}

}  // namespace moe
