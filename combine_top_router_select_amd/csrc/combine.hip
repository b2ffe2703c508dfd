// A5 - combine: weighted sum of the rows that served each token, back in
// token order.
//
// Sources: "Expert Coupling in MoE Pretraining" (summary), "The Communication
// Bottleneck": under expert parallelism each MoE layer dispatches rows to the
// experts and combines their outputs back.  "DODOCO" dataset card,
// "send_matrices.csv columns": combine moves the dispatch volumes in reverse;
// "Reading the counts": the payload is count x hidden x bytes per element of
// the dispatch precision (rows here are bf16, or fp8 E4M3 with bf16 output).
//
// Design: one wave per (token, row chunk).  Lanes j < k read slot_row[t][j]
// and the row weight; a slot whose row already appeared in an earlier slot is
// dropped (dedup rows serve several slots), negative rows are skipped, and each
// remaining lane learns the rank of its row among the token's distinct rows
// (DPP row shifts inside the 16-lane row that holds the slots).  The wave then
// issues the loads of every used row's chunk before any arithmetic (up to KMAX
// rows x NV vectors of 8 values in flight per lane: 16 bytes of bf16 or 8 bytes
// of fp8), accumulates in fp32 with fused multiply-adds over the rows in
// ascending row index starting from -0.0, and converts to bf16 with
// round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).  The order is fixed so
// that every output is a pure function of its inputs, bit for bit.  fp8 rows
// (OCP E4M3) are decoded with v_cvt_pk_f32_fp8, exact for every byte value.
// Row loads are nontemporal:
// each row is read once, so it should not displace cached data (measured:
// about 2 us less per 4096-token, top-6, hidden-2048 step).  So are the output
// stores of the combine proper (launch_combine_t gives the cases).
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

template <int NV, int KMAX, bool IN8, bool NTS>
__global__ void __launch_bounds__(256)
combine_kernel(const uint8_t* __restrict__ rows, const float* __restrict__ w,
               const int32_t* __restrict__ slot_row, int64_t T, int row_bytes, int k, int cpr,
               const int32_t* __restrict__ n_valid, uint8_t* __restrict__ out) {
  constexpr int OS = IN8 ? 2 : 1;
  const int lane = lane_id();
  const int64_t wid = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;
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

template <int NV, int KMAX, bool IN8>
static hipError_t launch_combine_t(const void* rows, const float* w, const int32_t* slot_row,
                                   int64_t T, int row_bytes, int k, const int32_t* n_valid,
                                   void* out, hipStream_t stream) {
  const int chunk = NV * kWave * InVec<IN8>::kBytes;
  const int cpr = (row_bytes + chunk - 1) / chunk;
  const int64_t blocks = (T * cpr + 3) / 4;
  const uint8_t* rb = static_cast<const uint8_t*>(rows);
  uint8_t* ob = static_cast<uint8_t*>(out);
  // Nontemporal output stores for the combine proper: nothing in the step
  // reads its output again, and keeping it out of the caches leaves the
  // Infinity Cache to the rows the next batch's kernels read (a 4096-token,
  // top-6, hidden-2048 step 42.0 -> 40.6 us).  Not for the receive-side
  // reduction (n_valid set), whose rows the combine reads next (16384-token
  // top-2 receive step 271 -> 282 us with them).
  if (n_valid == nullptr)
    hipLaunchKernelGGL((combine_kernel<NV, KMAX, IN8, true>), dim3(unsigned(blocks)), dim3(256),
                       0, stream, rb, w, slot_row, T, row_bytes, k, cpr, n_valid, ob);
  else
    hipLaunchKernelGGL((combine_kernel<NV, KMAX, IN8, false>), dim3(unsigned(blocks)), dim3(256),
                       0, stream, rb, w, slot_row, T, row_bytes, k, cpr, n_valid, ob);
  return hipGetLastError();
}

template <int KMAX, bool IN8>
static hipError_t launch_combine_k(const void* rows, const float* w, const int32_t* slot_row,
                                   int64_t T, int row_bytes, int k, const int32_t* n_valid,
                                   void* out, hipStream_t stream) {
  // keep KMAX * NV <= MOE_COMBINE_VECS input vectors in flight per lane
  const int vr = row_bytes / InVec<IN8>::kBytes;
  constexpr int NVCAP = 4;
  constexpr int NVB = MOE_COMBINE_VECS / KMAX > 0 ? MOE_COMBINE_VECS / KMAX : 1;
  constexpr int NVMAX = NVB < NVCAP ? NVB : NVCAP;
  if (NVMAX >= 4 && vr >= 4 * kWave)
    return launch_combine_t<(NVMAX >= 4 ? 4 : 1), KMAX, IN8>(rows, w, slot_row, T, row_bytes, k,
                                                              n_valid, out, stream);
  if (NVMAX >= 2 && vr >= 2 * kWave)
    return launch_combine_t<(NVMAX >= 2 ? 2 : 1), KMAX, IN8>(rows, w, slot_row, T, row_bytes, k,
                                                              n_valid, out, stream);
  return launch_combine_t<1, KMAX, IN8>(rows, w, slot_row, T, row_bytes, k, n_valid, out,
                                        stream);
}

template <bool IN8>
static hipError_t launch_combine_f(const void* rows, const float* w, const int32_t* slot_row,
                                   int64_t T, int row_bytes, int k, const int32_t* n_valid,
                                   void* out, hipStream_t stream) {
  if (k <= 1)
    return launch_combine_k<1, IN8>(rows, w, slot_row, T, row_bytes, k, n_valid, out, stream);
  if (k <= 2)
    return launch_combine_k<2, IN8>(rows, w, slot_row, T, row_bytes, k, n_valid, out, stream);
  if (k <= 4)
    return launch_combine_k<4, IN8>(rows, w, slot_row, T, row_bytes, k, n_valid, out, stream);
  if (k <= 6)
    return launch_combine_k<6, IN8>(rows, w, slot_row, T, row_bytes, k, n_valid, out, stream);
  if (k <= 8)
    return launch_combine_k<8, IN8>(rows, w, slot_row, T, row_bytes, k, n_valid, out, stream);
  return launch_combine_k<16, IN8>(rows, w, slot_row, T, row_bytes, k, n_valid, out, stream);
}

// row_bytes: bytes of one input row (H * 2 for bf16, H for fp8); the output
// rows are bf16 either way.  n_valid (device, may be null): only outputs
// t < *n_valid are computed and written (the receive-side reduction).
hipError_t launch_combine(const void* rows, const float* w, const int32_t* slot_row, int64_t T,
                          int row_bytes, int k, int in_fp8, const int32_t* n_valid, void* out,
                          hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (in_fp8)
    return launch_combine_f<true>(rows, w, slot_row, T, row_bytes, k, n_valid, out, stream);
  return launch_combine_f<false>(rows, w, slot_row, T, row_bytes, k, n_valid, out, stream);
}

}  // namespace moe
