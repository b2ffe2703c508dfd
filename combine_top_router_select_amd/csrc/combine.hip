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
#include "combine_rows.hpp"

namespace moe {

template <int NV, int KMAX, bool IN8, bool NTS>
__global__ void __launch_bounds__(256)
combine_kernel(const uint8_t* __restrict__ rows, const float* __restrict__ w,
               const int32_t* __restrict__ slot_row, int64_t T, int row_bytes, int k, int cpr,
               const int32_t* __restrict__ n_valid, uint8_t* __restrict__ out) {
  const int64_t wid = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;
  combine_unit<NV, KMAX, IN8, NTS>(rows, w, slot_row, T, row_bytes, k, cpr, n_valid, out, wid);
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
  constexpr int NVMAX = combine_nv_max<KMAX>();
  switch (combine_nv<KMAX, IN8>(row_bytes)) {
    case 4:
      return launch_combine_t<(NVMAX >= 4 ? 4 : 1), KMAX, IN8>(rows, w, slot_row, T, row_bytes,
                                                                k, n_valid, out, stream);
    case 2:
      return launch_combine_t<(NVMAX >= 2 ? 2 : 1), KMAX, IN8>(rows, w, slot_row, T, row_bytes,
                                                                k, n_valid, out, stream);
    default:
      return launch_combine_t<1, KMAX, IN8>(rows, w, slot_row, T, row_bytes, k, n_valid, out,
                                            stream);
  }
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
