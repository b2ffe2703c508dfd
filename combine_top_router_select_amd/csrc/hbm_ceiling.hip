// Reference kernels for the benchmark: the practical HBM ceilings that the
// dispatch and combine kernels are compared with.  Not part of the library's
// C ABI (include/moe_route.h); built into its own libmoe_hbm_ceiling.so, which
// only bench.py loads.
//
// Every kernel moves data in the dispatch kernel's pattern: one wave per
// 4 KiB chunk, 16-byte vector accesses, 1 KiB per wave instruction, every load
// of a chunk issued before the first store, nontemporal loads (each byte is
// read once).  What they leave out is what the method adds on top: the plan
// lookups and the metadata.
//   hbm_read     reads `bytes` (the XOR of each wave's words goes to a small
//                sink so the loads are not optimised away);
//   hbm_write    writes `bytes`;
//   hbm_copy     reads `bytes` and writes them elsewhere;
//   hbm_scatter  the dispatch's data movement with the positions given: row t
//                of x to rows pos[t][0..k-1] of dst;
//   hbm_scatter_distinct  the same with each distinct position of a token
//                written once (the deduplicating dispatch's rows, whose
//                positions repeat where several slots share a row);
//   hbm_gather_sum  the combine's data movement: out[t] = the fp32 sum, in
//                slot order, of the bf16 rows at token t's distinct positions,
//                truncated to bf16 (no weights, no ordering of the rows).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

#define HBM_API extern "C" __attribute__((visibility("default")))

namespace {

using moe::kWave;
using moe::u32x4;

constexpr int kNV = 4;                         // 16-byte vectors per lane per chunk
constexpr int64_t kChunk = kNV * kWave * 16;   // 4 KiB per wave
constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads)
read_kernel(const uint8_t* src, int64_t bytes, uint32_t* sink) {
  const int lane = moe::lane_id();
  const int64_t wid = (int64_t(blockIdx.x) * kThreads + threadIdx.x) / kWave;
  const int64_t base = wid * kChunk;
  u32x4 v[kNV];
#pragma unroll
  for (int i = 0; i < kNV; ++i) {
    int64_t off = base + int64_t(i * kWave + lane) * 16;
    off = off < bytes ? off : bytes - 16;
    v[i] = moe::load16_nt(src + off);
  }
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < kNV; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  if (x == 0x9E3779B9u) sink[wid & 255] = x;  // practically never taken; keeps the loads
}

__global__ void __launch_bounds__(kThreads)
write_kernel(uint8_t* dst, int64_t bytes) {
  const int lane = moe::lane_id();
  const int64_t wid = (int64_t(blockIdx.x) * kThreads + threadIdx.x) / kWave;
  const int64_t base = wid * kChunk;
  const u32x4 v = {uint32_t(wid), uint32_t(lane), 0u, 0u};
#pragma unroll
  for (int i = 0; i < kNV; ++i) {
    const int64_t off = base + int64_t(i * kWave + lane) * 16;
    if (off < bytes) moe::store16(dst + off, v);
  }
}

__global__ void __launch_bounds__(kThreads)
copy_kernel(const uint8_t* src, uint8_t* dst, int64_t bytes) {
  const int lane = moe::lane_id();
  const int64_t wid = (int64_t(blockIdx.x) * kThreads + threadIdx.x) / kWave;
  const int64_t base = wid * kChunk;
  u32x4 v[kNV];
#pragma unroll
  for (int i = 0; i < kNV; ++i) {
    int64_t off = base + int64_t(i * kWave + lane) * 16;
    off = off < bytes ? off : bytes - 16;
    v[i] = moe::load16_nt(src + off);
  }
#pragma unroll
  for (int i = 0; i < kNV; ++i) {
    const int64_t off = base + int64_t(i * kWave + lane) * 16;
    if (off < bytes) moe::store16(dst + off, v[i]);
  }
}

// One wave per (row, chunk): the chunk is read once and stored to each of
// the row's k destinations, or with DISTINCT to each distinct one (positions
// are assumed in range: they come from a dispatch of the same rows).
template <bool DISTINCT>
__global__ void __launch_bounds__(kThreads)
scatter_kernel(const uint8_t* x, const int32_t* __restrict__ pos, int64_t rows, int row_bytes,
               int k, int cpr, uint8_t* dst) {
  const int lane = moe::lane_id();
  const int64_t wid = (int64_t(blockIdx.x) * kThreads + threadIdx.x) / kWave;
  const int64_t t = wid / cpr;
  if (t >= rows) return;  // whole wave
  const int64_t c0 = (wid - t * cpr) * kChunk;
  const int p_lane = pos[t * k + (lane < k ? lane : k - 1)];
  // bit j set: slot j's position is stored (with DISTINCT, unless an earlier
  // slot of the token has the same position)
  uint64_t keep = k == 64 ? ~0ull : (1ull << k) - 1;
  if (DISTINCT) {
    bool dup = false;
    for (int j = 0; j < k; ++j) dup |= j < lane && moe::bcast(p_lane, j) == p_lane;
    keep &= __ballot(!dup);
  }
  u32x4 v[kNV];
#pragma unroll
  for (int i = 0; i < kNV; ++i) {
    int64_t off = c0 + int64_t(i * kWave + lane) * 16;
    off = off < row_bytes ? off : row_bytes - 16;
    v[i] = moe::load16_nt(x + t * row_bytes + off);
  }
  for (int j = 0; j < k; ++j) {
    if (!((keep >> j) & 1)) continue;  // uniform across the wave
    const int p = moe::bcast(p_lane, j);
    uint8_t* d = dst + int64_t(p) * row_bytes + c0;
#pragma unroll
    for (int i = 0; i < kNV; ++i) {
      const int64_t off = int64_t(i * kWave + lane) * 16;
      if (c0 + off < row_bytes) moe::store16(d + off, v[i]);
    }
  }
}

// One wave per (token, chunk): the chunks of all K slots' rows are loaded
// before the first add (K x NV vectors in flight per lane; a repeated
// position is loaded again: loads under a branch would each wait), and the
// sum takes each distinct row once.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
}

template <int NV, int K>
__global__ void __launch_bounds__(kThreads)
gather_sum_kernel(const uint8_t* rows, const int32_t* __restrict__ pos, int64_t tokens,
                  int row_bytes, int cpr, uint8_t* out) {
  const int lane = moe::lane_id();
  const int64_t wid = (int64_t(blockIdx.x) * kThreads + threadIdx.x) / kWave;
  const int64_t t = wid / cpr;
  if (t >= tokens) return;  // whole wave
  const int64_t c0 = (wid - t * cpr) * (NV * kWave * 16);
  const int p_lane = pos[t * K + (lane < K ? lane : K - 1)];
  u32x4 v[K][NV];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const uint8_t* row = rows + int64_t(moe::bcast(p_lane, j)) * row_bytes;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int64_t off = c0 + int64_t(i * kWave + lane) * 16;
      off = off < row_bytes ? off : row_bytes - 16;
      v[j][i] = moe::load16_nt(row + off);
    }
  }
  bool dup = false;
#pragma unroll
  for (int j = 0; j < K; ++j) dup |= j < lane && moe::bcast(p_lane, j) == p_lane;
  const uint64_t keep = __ballot(!dup);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if (!((keep >> j) & 1)) continue;  // uniform across the wave
      const u32x4 q = v[j][i];
      a[0] += bf16_lo(q.x); a[1] += bf16_hi(q.x); a[2] += bf16_lo(q.y); a[3] += bf16_hi(q.y);
      a[4] += bf16_lo(q.z); a[5] += bf16_hi(q.z); a[6] += bf16_lo(q.w); a[7] += bf16_hi(q.w);
    }
    const u32x4 o = {bf16_pair(a[0], a[1]), bf16_pair(a[2], a[3]), bf16_pair(a[4], a[5]),
                     bf16_pair(a[6], a[7])};
    const int64_t off = c0 + int64_t(i * kWave + lane) * 16;
    if (off < row_bytes) moe::store16_nt(out + t * row_bytes + off, o);
  }
}

template <int K>
int launch_gather_sum(const void* rows, const int32_t* pos, int64_t tokens, int row_bytes,
                      void* out, hipStream_t stream) {
  constexpr int NV = K <= 6 ? 4 : (K <= 12 ? 2 : 1);  // at most 24 vectors in flight
  const int cpr = (row_bytes + NV * kWave * 16 - 1) / (NV * kWave * 16);
  const int64_t waves = tokens * cpr;
  const unsigned grid = unsigned((waves + kThreads / kWave - 1) / (kThreads / kWave));
  hipLaunchKernelGGL((gather_sum_kernel<NV, K>), dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const uint8_t*>(rows), pos, tokens, row_bytes, cpr,
                     static_cast<uint8_t*>(out));
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

unsigned grid_for(int64_t bytes) {
  const int64_t waves = (bytes + kChunk - 1) / kChunk;
  return unsigned((waves + kThreads / kWave - 1) / (kThreads / kWave));
}

int status(hipError_t e) { return e == hipSuccess ? 0 : 1; }

}  // namespace

// Each returns 0, or 1 when the launch failed; 2 for invalid sizes (bytes or
// row_bytes not a positive multiple of 16, k outside 1..64).
HBM_API int hbm_read(const void* src, int64_t bytes, void* sink, void* stream) {
  if (bytes < 16 || bytes % 16 != 0 || !src || !sink) return 2;
  hipLaunchKernelGGL(read_kernel, dim3(grid_for(bytes)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(src), bytes,
                     static_cast<uint32_t*>(sink));
  return status(hipGetLastError());
}

HBM_API int hbm_write(void* dst, int64_t bytes, void* stream) {
  if (bytes < 16 || bytes % 16 != 0 || !dst) return 2;
  hipLaunchKernelGGL(write_kernel, dim3(grid_for(bytes)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint8_t*>(dst), bytes);
  return status(hipGetLastError());
}

HBM_API int hbm_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 16 || bytes % 16 != 0 || !src || !dst) return 2;
  hipLaunchKernelGGL(copy_kernel, dim3(grid_for(bytes)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(src),
                     static_cast<uint8_t*>(dst), bytes);
  return status(hipGetLastError());
}

static int scatter(bool distinct, const void* x, const int32_t* pos, int64_t rows, int row_bytes,
                   int k, void* dst, void* stream) {
  if (rows < 1 || row_bytes < 16 || row_bytes % 16 != 0 || k < 1 || k > 64 || !x || !pos ||
      !dst)
    return 2;
  const int cpr = int((row_bytes + kChunk - 1) / kChunk);
  const int64_t waves = rows * cpr;
  const unsigned grid = unsigned((waves + kThreads / kWave - 1) / (kThreads / kWave));
  auto kern = distinct ? scatter_kernel<true> : scatter_kernel<false>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t*>(x), pos, rows, row_bytes, k, cpr,
                     static_cast<uint8_t*>(dst));
  return status(hipGetLastError());
}

HBM_API int hbm_scatter(const void* x, const int32_t* pos, int64_t rows, int row_bytes, int k,
                        void* dst, void* stream) {
  return scatter(false, x, pos, rows, row_bytes, k, dst, stream);
}

HBM_API int hbm_scatter_distinct(const void* x, const int32_t* pos, int64_t rows, int row_bytes,
                                 int k, void* dst, void* stream) {
  return scatter(true, x, pos, rows, row_bytes, k, dst, stream);
}

// rows: bf16 rows of row_bytes bytes; pos [tokens][k] row indices (assumed in
// range: they come from a dispatch of the same rows); out [tokens][row_bytes].
// 2 for invalid sizes (row_bytes not a positive multiple of 16, k outside
// 1..16, no tokens).
HBM_API int hbm_gather_sum(const void* rows, const int32_t* pos, int64_t tokens, int row_bytes,
                           int k, void* out, void* stream) {
  if (tokens < 1 || row_bytes < 16 || row_bytes % 16 != 0 || k < 1 || k > 16 || !rows || !pos ||
      !out)
    return 2;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (k) {
#define MOE_GS(K) \
  case K: return launch_gather_sum<K>(rows, pos, tokens, row_bytes, out, s);
    MOE_GS(1) MOE_GS(2) MOE_GS(3) MOE_GS(4) MOE_GS(5) MOE_GS(6) MOE_GS(7) MOE_GS(8)
    MOE_GS(9) MOE_GS(10) MOE_GS(11) MOE_GS(12) MOE_GS(13) MOE_GS(14) MOE_GS(15) MOE_GS(16)
#undef MOE_GS
    default: return 2;
  }
}

// Host: properties of the current device: compute units, memory clock (kHz),
// memory bus width (bits), shader clock (kHz), and the architecture name
// (e.g. gfx950) into arch[arch_len].  Returns 0, or 1 on a HIP error.
HBM_API int hbm_device_info(int* cu_count, int* mem_clock_khz, int* mem_bus_width,
                            int* clock_khz, char* arch, int arch_len) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) return 1;
  *cu_count = p.multiProcessorCount;
  *mem_clock_khz = p.memoryClockRate;
  *mem_bus_width = p.memoryBusWidth;
  *clock_khz = p.clockRate;
  int i = 0;
  for (; i + 1 < arch_len && p.gcnArchName[i] != '\0'; ++i) arch[i] = p.gcnArchName[i];
  if (arch_len > 0) arch[i] = '\0';
  return 0;
}
