// Plain dispatch without a caller-supplied workspace: for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops that
// forbid allocation, harnesses without an allocator).  The dispatch plan that
// moe_send_counts() would leave in the caller's workspace goes to one static
// scratch array per device instead.
#include <hip/hip_runtime.h>

#include <mutex>

#include "common.hpp"
#include "moe_route.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace moe {
hipError_t launch_send_counts(const int32_t*, int64_t, int, int, int, const int32_t*, int,
                              int32_t*, int32_t*, int32_t*, int32_t*, void*, hipStream_t);
hipError_t launch_dispatch(const void*, const int32_t*, const float*, int64_t, int, int, int,
                           int, const void*, int, void*, int32_t*, int32_t*, float*, float*,
                           int32_t*, int32_t*, int64_t, int32_t*, hipStream_t);
}  // namespace moe

// The plan scratch: every GPU the library runs on holds one copy until the
// process ends.  Host code never passes `scratch` itself to a kernel (on the
// host the name stands for a host-side shadow, not a device address); it uses
// the device address that hipGetSymbolAddress() returns for the current device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up once per device
// (with that device current) and kept.  nullptr on a HIP error.
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  try {  // no exception leaves the ABI (a failed lock reads as a HIP error)
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
      void* ptr = nullptr;
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
      g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
  } catch (...) {
    return nullptr;
  }
}

}  // namespace

MOE_API int moe_dispatch_permute_noalloc(const void* x, const int32_t* topk_idx,
                                         const float* topk_gate, int64_t tokens, int hidden_dim,
                                         int n_experts, int top_k, int n_ranks,
                                         const int32_t* placement, int bytes_per_element,
                                         int32_t* expert_counts, int32_t* rank_counts,
                                         int32_t* rank_offsets, int32_t* expert_offsets,
                                         void* send, int32_t* row_token, int32_t* row_expert,
                                         float* row_weight, int32_t* slot_row, void* stream) {
  // the argument checks of moe_send_counts() and moe_dispatch_permute()
  const size_t need = moe_workspace_bytes(tokens, n_experts, top_k, n_ranks, 0);
  if (tokens < 0 || n_experts < 1 || top_k < 1 || top_k > n_experts || n_ranks < 1 ||
      n_experts % n_ranks != 0 || hidden_dim < 1 || bytes_per_element < 1)
    return MOE_EINVAL;
  if (need == 0) return MOE_EUNSUPPORTED;  // outside the limits of moe_workspace_bytes()
  if (bytes_per_element != 1 && bytes_per_element != 2 && bytes_per_element != 4)
    return MOE_EUNSUPPORTED;
  const int64_t rb = int64_t(hidden_dim) * bytes_per_element;
  if (rb % 16 != 0 || rb > INT32_MAX / 2) return MOE_EUNSUPPORTED;
  if (need > size_t(MOE_NOALLOC_SCRATCH_BYTES)) return MOE_EUNSUPPORTED;  // plan too big
  if (!expert_counts || !rank_counts || !rank_offsets) return MOE_EINVAL;
  if (tokens > 0 && (!x || !topk_idx || !topk_gate || !send || !row_token || !row_expert ||
                     !row_weight || !slot_row))
    return MOE_EINVAL;
  void* ws = scratch_for_current_device();
  if (ws == nullptr) return MOE_EHIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err = moe::launch_send_counts(topk_idx, tokens, n_experts, top_k, n_ranks, placement,
                                           0, expert_counts, rank_counts, rank_offsets,
                                           expert_offsets, ws, st);
  if (err != hipSuccess) return MOE_EHIP;
  if (tokens == 0) return MOE_OK;
  err = moe::launch_dispatch(x, topk_idx, topk_gate, tokens, int(rb), n_experts, top_k, n_ranks,
                             ws, 0, send, row_token, row_expert, nullptr, row_weight, slot_row,
                             nullptr, 0, nullptr, st);
  return err == hipSuccess ? MOE_OK : MOE_EHIP;
}
