// A5 - combine: weighted sum of the rows that served each token, back in
// token order.
//
// Sources: "Expert Coupling in MoE Pretraining" (summary), "The Communication
// Bottleneck": under expert parallelism each MoE layer dispatches rows to the
// experts and combines their outputs back.  "DODOCO" dataset card,
// "send_matrices.csv columns": combine moves the dispatch volumes in reverse.
//
// Design: one wave per (token, row chunk).  Lanes j < k read slot_row[t][j]
// and the row weight; a slot whose row already appeared in an earlier slot is
// dropped (dedup rows serve several slots), negative rows are skipped.  The
// wave then issues the loads of every used row's chunk before any arithmetic
// (KMAX rows x NV 16-byte vectors in flight per lane), accumulates in fp32
// with fused multiply-adds in slot order starting from -0.0, and converts to
// bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).  Row loads are
// nontemporal: each row is read once, so it should not displace cached data
// (measured: about 2 us less per 4096-token, top-6, hidden-2048 step).
#include "common.hpp"

#ifndef MOE_COMBINE_NT
#define MOE_COMBINE_NT 1
#endif

namespace moe {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 f = {lo, hi};
  const bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

// The weighted sum of a token's rows for one chunk: NQ >= nrows rows are
// loaded (all loads before any arithmetic; rows past nrows repeat the first
// one and are not added), accumulated in fp32 from -0.0 in slot order, and
// stored as bf16.
template <int NQ, int NV>
__device__ __forceinline__ void sum_rows(const uint8_t* __restrict__ rows, int row_bytes,
                                         int64_t chunk0, uint64_t um, int j0, int nrows, int rr,
                                         float wr, int lane, uint8_t* __restrict__ dst) {
  u32x4 y[NQ][NV];
  float wq[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    int j = j0;
    if (q < nrows) {
      j = __ffsll((unsigned long long)um) - 1;
      um &= um - 1;
    }
    const int p = bcast(rr, j);
    wq[q] = bcastf(wr, j);
    const uint8_t* src = rows + int64_t(p) * row_bytes;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int64_t off = chunk0 + int64_t(i * kWave + lane) * 16;
      off = off < row_bytes ? off : row_bytes - 16;
      y[q][i] = MOE_COMBINE_NT ? load16_nt(src + off) : load16(src + off);
    }
  }
  float acc[NV][8];
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int h = 0; h < 8; ++h) acc[i][h] = -0.0f;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    if (q < nrows) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const uint32_t u = y[q][i][h];
          acc[i][2 * h] = __builtin_fmaf(wq[q], __uint_as_float(u << 16), acc[i][2 * h]);
          acc[i][2 * h + 1] =
              __builtin_fmaf(wq[q], __uint_as_float(u & 0xFFFF0000u), acc[i][2 * h + 1]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int64_t off = chunk0 + int64_t(i * kWave + lane) * 16;
    if (off < row_bytes) {
      u32x4 o;
#pragma unroll
      for (int h = 0; h < 4; ++h) o[h] = pack_bf16x2(acc[i][2 * h], acc[i][2 * h + 1]);
      store16(dst + off, o);
    }
  }
}

template <int NV, int KMAX>
__global__ void __launch_bounds__(256)
combine_kernel(const uint8_t* __restrict__ rows, const float* __restrict__ w,
               const int32_t* __restrict__ slot_row, int64_t T, int row_bytes, int k, int cpr,
               const int32_t* __restrict__ n_valid, uint8_t* __restrict__ out) {
  const int lane = lane_id();
  const int64_t wid = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;
  const int64_t t = wid / cpr;
  const int c = int(wid - t * cpr);
  if (t >= T) return;  // whole wave
  if (n_valid && t >= *n_valid) return;  // whole wave: only the first *n_valid outputs
  const int64_t chunk0 = int64_t(c) * (NV * kWave * 16);
  // All loads are unconditional from clamped, in-bounds addresses (a load under
  // a branch is followed by a wait for it); only arithmetic and stores are
  // predicated.
  const int jl = lane < k ? lane : k - 1;
  const int r_raw = slot_row[t * k + jl];
  const int r = lane < k ? r_raw : -1;
  bool use = r >= 0;
  for (int i = 0; i < k; ++i) {
    const int ri = bcast(r, i);
    if (i < lane && ri == r) use = false;
  }
  uint64_t um = __ballot(use);
  const int nrows = __popcll(um);
  uint8_t* dst = out + t * row_bytes;
  if (nrows == 0) {  // no row serves this token: the empty sum, -0.0
    const u32x4 nz = {0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int64_t off = chunk0 + int64_t(i * kWave + lane) * 16;
      if (off < row_bytes) store16(dst + off, nz);
    }
    return;
  }
  const int j0 = __ffsll((unsigned long long)um) - 1;
  const int rr = use ? r : bcast(r, j0);  // every lane names a valid row
  const float wr = w ? w[rr] : 1.0f;
  // as few row loads as the token needs (nrows is wave-uniform): a token served
  // by one or two rows - most received rows in the reduction - does not load
  // KMAX rows
  if constexpr (KMAX >= 1) {
    if (nrows <= 1)
      return sum_rows<1, NV>(rows, row_bytes, chunk0, um, j0, nrows, rr, wr, lane, dst);
  }
  if constexpr (KMAX >= 2) {
    if (nrows <= 2)
      return sum_rows<2, NV>(rows, row_bytes, chunk0, um, j0, nrows, rr, wr, lane, dst);
  }
  if constexpr (KMAX > 4) {
    if (nrows <= 4)
      return sum_rows<4, NV>(rows, row_bytes, chunk0, um, j0, nrows, rr, wr, lane, dst);
  }
  sum_rows<KMAX, NV>(rows, row_bytes, chunk0, um, j0, nrows, rr, wr, lane, dst);
}

template <int NV, int KMAX>
static hipError_t launch_combine_t(const void* rows, const float* w, const int32_t* slot_row,
                                   int64_t T, int row_bytes, int k, const int32_t* n_valid,
                                   void* out, hipStream_t stream) {
  const int chunk = NV * kWave * 16;
  const int cpr = (row_bytes + chunk - 1) / chunk;
  const int64_t blocks = (T * cpr + 3) / 4;
  hipLaunchKernelGGL((combine_kernel<NV, KMAX>), dim3(unsigned(blocks)), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(rows), w, slot_row, T, row_bytes, k, cpr,
                     n_valid, static_cast<uint8_t*>(out));
  return hipGetLastError();
}

template <int KMAX>
static hipError_t launch_combine_k(const void* rows, const float* w, const int32_t* slot_row,
                                   int64_t T, int row_bytes, int k, const int32_t* n_valid,
                                   void* out, hipStream_t stream) {
  // keep KMAX * NV <= 32 vectors (128 VGPRs) in flight per lane
  const int vr = row_bytes / 16;
  constexpr int NVMAX = (32 / KMAX) < 4 ? (32 / KMAX) : 4;
  if (NVMAX >= 4 && vr >= 4 * kWave)
    return launch_combine_t<(NVMAX >= 4 ? 4 : 1), KMAX>(rows, w, slot_row, T, row_bytes, k,
                                                         n_valid, out, stream);
  if (NVMAX >= 2 && vr >= 2 * kWave)
    return launch_combine_t<(NVMAX >= 2 ? 2 : 1), KMAX>(rows, w, slot_row, T, row_bytes, k,
                                                         n_valid, out, stream);
  return launch_combine_t<1, KMAX>(rows, w, slot_row, T, row_bytes, k, n_valid, out, stream);
}

// n_valid (device, may be null): only outputs t < *n_valid are computed and
// written (the receive-side reduction over the received rows).
hipError_t launch_combine(const void* rows, const float* w, const int32_t* slot_row, int64_t T,
                          int row_bytes, int k, const int32_t* n_valid, void* out,
                          hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (k <= 1) return launch_combine_k<1>(rows, w, slot_row, T, row_bytes, k, n_valid, out, stream);
  if (k <= 2) return launch_combine_k<2>(rows, w, slot_row, T, row_bytes, k, n_valid, out, stream);
  if (k <= 4) return launch_combine_k<4>(rows, w, slot_row, T, row_bytes, k, n_valid, out, stream);
  if (k <= 6) return launch_combine_k<6>(rows, w, slot_row, T, row_bytes, k, n_valid, out, stream);
  if (k <= 8) return launch_combine_k<8>(rows, w, slot_row, T, row_bytes, k, n_valid, out, stream);
  return launch_combine_k<16>(rows, w, slot_row, T, row_bytes, k, n_valid, out, stream);
}

}  // namespace moe
