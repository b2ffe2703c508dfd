// C ABI of libmoe_route.so: host-side argument checks, then launches on the
// caller's stream.  Everything that can be checked without reading device
// memory is checked here, before anything is enqueued.
#include <limits.h>

#include "common.hpp"
#include "moe_route.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace moe {
hipError_t launch_route_topk(const float*, int64_t, int, int, int, int32_t*, float*, hipStream_t);
hipError_t launch_send_counts(const int32_t*, int64_t, int, int, int, const int32_t*, int,
                              int32_t*, int32_t*, int32_t*, int32_t*, void*, hipStream_t);
hipError_t launch_dispatch(const void*, const int32_t*, const float*, int64_t, int, int, int,
                           int, const void*, int, void*, int32_t*, int32_t*, float*, float*,
                           int32_t*, int32_t*, int64_t, int32_t*, hipStream_t);
hipError_t launch_combine(const void*, const float*, const int32_t*, int64_t, int, int, int,
                          const int32_t*, void*, hipStream_t);
hipError_t launch_expand_counts(const int32_t*, int64_t, int, int, int, const int32_t*,
                                const int32_t*, int32_t*, int32_t*, int32_t*, int32_t*, void*,
                                hipStream_t);
hipError_t launch_expand(const void*, const float*, const int32_t*, int64_t, int, int, int, int,
                         const void*, void*, int64_t, int32_t*, int32_t*, float*, int32_t*,
                         hipStream_t);
int placement_search(const int32_t*, int, int, const int32_t*, int, int32_t*, int64_t*, int*);
hipError_t launch_shuffle_fit(const int32_t*, const int32_t*, const int32_t*, int64_t, int, int,
                              int, const int32_t*, int32_t*, int32_t*, hipStream_t);
hipError_t launch_shuffle_predict(const int32_t*, const int32_t*, int64_t, int, int, int,
                                  const int32_t*, const int32_t*, int, float*, hipStream_t);
int shuffle_assign(const float*, int64_t, int, int32_t*);
hipError_t launch_coselect(const int32_t*, int64_t, int, int, int32_t*, hipStream_t);
hipError_t launch_route_plan(const float*, int64_t, int, int, int, int, const int32_t*, int,
                             int32_t*, float*, int32_t*, int32_t*, int32_t*, int32_t*, int64_t,
                             int32_t*, void*, hipStream_t);
bool route_tiles_fit(int64_t, int);
hipError_t launch_route_tiles(const float*, int64_t, int, int, int, int, const int32_t*, int,
                              int32_t*, float*, void*, hipStream_t);
bool dispatch_scans_plan(int64_t, int, int, int, int, int);
hipError_t launch_dispatch_scan(const void*, const int32_t*, const float*, int64_t, int, int, int,
                                int, const int32_t*, void*, int, void*, int32_t*, int32_t*,
                                float*, float*, int32_t*, int32_t*, int32_t*, int32_t*, int32_t*,
                                int32_t*, int64_t, int32_t*, hipStream_t);
hipError_t launch_plan_scan(int64_t, int, int, int, const int32_t*, int, int32_t*, int32_t*,
                            int32_t*, int32_t*, void*, hipStream_t);
hipError_t launch_combine_route(const void*, const float*, const int32_t*, int64_t, int, int, int,
                                void*, const float*, int64_t, int, int, int, int, const int32_t*,
                                int, int32_t*, float*, void*, hipStream_t);
}  // namespace moe

namespace {

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// tokens, experts and top_k: shared by every entry point.
int check_tek(int64_t tokens, int n_experts, int top_k) {
  if (tokens < 0 || n_experts < 1 || top_k < 1 || top_k > n_experts) return MOE_EINVAL;
  if (n_experts > MOE_MAX_EXPERTS || top_k > MOE_MAX_TOP_K) return MOE_EUNSUPPORTED;
  if (tokens > int64_t(INT_MAX) / top_k) return MOE_EUNSUPPORTED;  // rows indexed by int32
  return MOE_OK;
}

int check_ranks(int n_experts, int n_ranks) {
  if (n_ranks < 1 || n_experts % n_ranks != 0) return MOE_EINVAL;
  if (n_ranks > MOE_MAX_RANKS) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

int check_rows(int hidden_dim, int bytes_per_element) {
  if (hidden_dim < 1 || bytes_per_element < 1) return MOE_EINVAL;
  if (bytes_per_element != 1 && bytes_per_element != 2 && bytes_per_element != 4)
    return MOE_EUNSUPPORTED;
  const int64_t rb = int64_t(hidden_dim) * bytes_per_element;
  if (rb % 16 != 0 || rb > INT_MAX / 2) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

}  // namespace

MOE_API const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK: success";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: outside the library's supported limits";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace smaller than moe_workspace_bytes()";
    case MOE_EHIP: return "MOE_EHIP: a HIP launch failed";
    default: return "unknown moe_route status";
  }
}

MOE_API size_t moe_workspace_bytes(int64_t tokens, int n_experts, int top_k, int n_ranks,
                                   int dedup) {
  if (check_tek(tokens, n_experts, top_k) != MOE_OK) return 0;
  if (check_ranks(n_experts, n_ranks) != MOE_OK) return 0;
  return moe::plan_layout(tokens, n_experts, top_k, n_ranks, dedup ? 1 : 0).bytes;
}

MOE_API int moe_route_topk(const float* logits, int64_t tokens, int n_experts, int top_k,
                           int32_t* topk_idx, float* topk_gate, void* stream) {
  int st = check_tek(tokens, n_experts, top_k);
  if (st != MOE_OK) return st;
  if (tokens == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_gate) return MOE_EINVAL;
  return hip_status(moe::launch_route_topk(logits, tokens, n_experts, top_k, 0, topk_idx,
                                           topk_gate, as_stream(stream)));
}

MOE_API int moe_route_topk_softmax_all(const float* logits, int64_t tokens, int n_experts,
                                       int top_k, int32_t* topk_idx, float* topk_gate,
                                       void* stream) {
  int st = check_tek(tokens, n_experts, top_k);
  if (st != MOE_OK) return st;
  if (tokens == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_gate) return MOE_EINVAL;
  return hip_status(moe::launch_route_topk(logits, tokens, n_experts, top_k, 1, topk_idx,
                                           topk_gate, as_stream(stream)));
}

MOE_API int moe_send_counts(const int32_t* topk_idx, int64_t tokens, int n_experts, int top_k,
                            int n_ranks, const int32_t* placement, int dedup,
                            int32_t* expert_counts, int32_t* rank_counts,
                            int32_t* rank_offsets, int32_t* expert_offsets, void* workspace,
                            size_t workspace_bytes, void* stream) {
  int st = check_tek(tokens, n_experts, top_k);
  if (st != MOE_OK) return st;
  if ((st = check_ranks(n_experts, n_ranks)) != MOE_OK) return st;
  if ((tokens > 0 && !topk_idx) || !expert_counts || !rank_counts || !rank_offsets || !workspace)
    return MOE_EINVAL;
  if (workspace_bytes < moe_workspace_bytes(tokens, n_experts, top_k, n_ranks, dedup))
    return MOE_EWORKSPACE;
  return hip_status(moe::launch_send_counts(topk_idx, tokens, n_experts, top_k, n_ranks,
                                            placement, dedup ? 1 : 0, expert_counts,
                                            rank_counts, rank_offsets,
                                            dedup ? nullptr : expert_offsets, workspace,
                                            as_stream(stream)));
}

MOE_API int moe_route_plan(const float* logits, int64_t tokens, int n_experts, int top_k,
                           int gating, int n_ranks, const int32_t* placement, int dedup,
                           int32_t* topk_idx, float* topk_gate, int32_t* expert_counts,
                           int32_t* rank_counts, int32_t* rank_offsets, int32_t* expert_offsets,
                           int64_t coselect_tokens, int32_t* coselect, void* workspace,
                           size_t workspace_bytes, void* stream) {
  int st = check_tek(tokens, n_experts, top_k);
  if (st != MOE_OK) return st;
  if ((st = check_ranks(n_experts, n_ranks)) != MOE_OK) return st;
  if (gating != 0 && gating != 1) return MOE_EINVAL;
  if (coselect_tokens < 0 || coselect_tokens > tokens || (coselect_tokens > 0 && !coselect))
    return MOE_EINVAL;
  if ((tokens > 0 && (!logits || !topk_idx || !topk_gate)) || !expert_counts || !rank_counts ||
      !rank_offsets || !workspace)
    return MOE_EINVAL;
  if (workspace_bytes < moe_workspace_bytes(tokens, n_experts, top_k, n_ranks, dedup))
    return MOE_EWORKSPACE;
  return hip_status(moe::launch_route_plan(logits, tokens, n_experts, top_k, gating, n_ranks,
                                           placement, dedup ? 1 : 0, topk_idx, topk_gate,
                                           expert_counts, rank_counts, rank_offsets,
                                           dedup ? nullptr : expert_offsets, coselect_tokens,
                                           coselect, workspace, as_stream(stream)));
}

MOE_API int moe_dispatch_permute(const void* x, const int32_t* topk_idx, const float* topk_gate,
                                 int64_t tokens, int hidden_dim, int n_experts, int top_k,
                                 int n_ranks, int bytes_per_element, const void* workspace,
                                 size_t workspace_bytes, void* send, int32_t* row_token,
                                 int32_t* row_expert, float* row_weight, int32_t* slot_row,
                                 int64_t coselect_tokens, int32_t* coselect, void* stream) {
  int st = check_tek(tokens, n_experts, top_k);
  if (st != MOE_OK) return st;
  if ((st = check_ranks(n_experts, n_ranks)) != MOE_OK) return st;
  if ((st = check_rows(hidden_dim, bytes_per_element)) != MOE_OK) return st;
  if (!workspace) return MOE_EINVAL;
  if (coselect && (coselect_tokens < 0 || coselect_tokens > tokens)) return MOE_EINVAL;
  if (workspace_bytes < moe_workspace_bytes(tokens, n_experts, top_k, n_ranks, 0))
    return MOE_EWORKSPACE;
  if (tokens == 0) return MOE_OK;
  if (!x || !topk_idx || !topk_gate || !send || !row_token || !row_expert || !row_weight ||
      !slot_row)
    return MOE_EINVAL;
  return hip_status(moe::launch_dispatch(x, topk_idx, topk_gate, tokens,
                                         hidden_dim * bytes_per_element, n_experts, top_k,
                                         n_ranks, workspace, 0, send, row_token,
                                         row_expert, nullptr, row_weight, slot_row, nullptr,
                                         coselect ? coselect_tokens : 0, coselect,
                                         as_stream(stream)));
}

MOE_API int moe_dispatch_permute_dedup(const void* x, const int32_t* topk_idx,
                                       const float* topk_gate, int64_t tokens, int hidden_dim,
                                       int n_experts, int top_k, int n_ranks,
                                       int bytes_per_element, const void* workspace,
                                       size_t workspace_bytes, void* send, int32_t* row_token,
                                       int32_t* row_experts, float* row_gates,
                                       float* row_weight, int32_t* slot_row, int32_t* n_rows,
                                       int64_t coselect_tokens, int32_t* coselect,
                                       void* stream) {
  int st = check_tek(tokens, n_experts, top_k);
  if (st != MOE_OK) return st;
  if ((st = check_ranks(n_experts, n_ranks)) != MOE_OK) return st;
  if ((st = check_rows(hidden_dim, bytes_per_element)) != MOE_OK) return st;
  if (!workspace || !n_rows) return MOE_EINVAL;
  if (coselect && (coselect_tokens < 0 || coselect_tokens > tokens)) return MOE_EINVAL;
  if (workspace_bytes < moe_workspace_bytes(tokens, n_experts, top_k, n_ranks, 1))
    return MOE_EWORKSPACE;
  if (tokens > 0 && (!x || !topk_idx || !topk_gate || !send || !row_token || !row_experts ||
                     !row_gates || !row_weight || !slot_row))
    return MOE_EINVAL;
  return hip_status(moe::launch_dispatch(x, topk_idx, topk_gate, tokens,
                                         hidden_dim * bytes_per_element, n_experts, top_k,
                                         n_ranks, workspace, 1, send, row_token,
                                         row_experts, row_gates, row_weight, slot_row, n_rows,
                                         coselect ? coselect_tokens : 0, coselect,
                                         as_stream(stream)));
}

MOE_API int moe_route_dispatch(const float* logits, const void* x, int64_t tokens, int hidden_dim,
                               int n_experts, int top_k, int gating, int n_ranks,
                               const int32_t* placement, int dedup, int bytes_per_element,
                               int32_t* topk_idx, float* topk_gate, int32_t* expert_counts,
                               int32_t* rank_counts, int32_t* rank_offsets,
                               int32_t* expert_offsets, void* send, int32_t* row_token,
                               int32_t* row_experts, float* row_gates, float* row_weight,
                               int32_t* slot_row, int32_t* n_rows, int64_t coselect_tokens,
                               int32_t* coselect, void* workspace, size_t workspace_bytes,
                               void* stream) {
  int st = check_tek(tokens, n_experts, top_k);
  if (st != MOE_OK) return st;
  if ((st = check_ranks(n_experts, n_ranks)) != MOE_OK) return st;
  if ((st = check_rows(hidden_dim, bytes_per_element)) != MOE_OK) return st;
  if (gating != 0 && gating != 1) return MOE_EINVAL;
  if (coselect && (coselect_tokens < 0 || coselect_tokens > tokens)) return MOE_EINVAL;
  if (!expert_counts || !rank_counts || !rank_offsets || !workspace || (dedup && !n_rows))
    return MOE_EINVAL;
  if (tokens > 0 && (!logits || !x || !topk_idx || !topk_gate || !send || !row_token ||
                     !row_experts || !row_weight || !slot_row || (dedup && !row_gates)))
    return MOE_EINVAL;
  const int d = dedup ? 1 : 0;
  if (workspace_bytes < moe_workspace_bytes(tokens, n_experts, top_k, n_ranks, d))
    return MOE_EWORKSPACE;
  const int rb = hidden_dim * bytes_per_element;
  const int64_t ncs = coselect ? coselect_tokens : 0;
  int32_t* eo = d ? nullptr : expert_offsets;
  hipStream_t s = as_stream(stream);
  if (moe::route_tiles_fit(tokens, n_experts) &&
      moe::dispatch_scans_plan(tokens, n_experts, top_k, n_ranks, d, rb)) {
    // two launches: routing with the tile counts, then the dispatch, whose
    // workgroups scan the plan themselves
    if (moe::launch_route_tiles(logits, tokens, n_experts, top_k, gating, n_ranks, placement, d,
                                topk_idx, topk_gate, workspace, s) != hipSuccess)
      return MOE_EHIP;
    return hip_status(moe::launch_dispatch_scan(
        x, topk_idx, topk_gate, tokens, rb, n_experts, top_k, n_ranks, placement, workspace, d,
        send, row_token, row_experts, d ? row_gates : nullptr, row_weight, slot_row,
        d ? n_rows : nullptr, expert_counts, rank_counts, rank_offsets, eo, ncs, coselect, s));
  }
  // larger plans: the routing call with its scan, then the dispatch
  if (moe::launch_route_plan(logits, tokens, n_experts, top_k, gating, n_ranks, placement, d,
                             topk_idx, topk_gate, expert_counts, rank_counts, rank_offsets, eo, 0,
                             nullptr, workspace, s) != hipSuccess)
    return MOE_EHIP;
  if (tokens == 0 && !d) return MOE_OK;
  return hip_status(moe::launch_dispatch(x, topk_idx, topk_gate, tokens, rb, n_experts, top_k,
                                         n_ranks, workspace, d, send, row_token, row_experts,
                                         d ? row_gates : nullptr, row_weight, slot_row,
                                         d ? n_rows : nullptr, ncs, coselect, s));
}

MOE_API int moe_dispatch_routed(const void* x, const int32_t* topk_idx, const float* topk_gate,
                                int64_t tokens, int hidden_dim, int n_experts, int top_k,
                                int n_ranks, const int32_t* placement, int dedup,
                                int bytes_per_element, int32_t* expert_counts,
                                int32_t* rank_counts, int32_t* rank_offsets,
                                int32_t* expert_offsets, void* send, int32_t* row_token,
                                int32_t* row_experts, float* row_gates, float* row_weight,
                                int32_t* slot_row, int32_t* n_rows, int64_t coselect_tokens,
                                int32_t* coselect, void* workspace, size_t workspace_bytes,
                                void* stream) {
  int st = check_tek(tokens, n_experts, top_k);
  if (st != MOE_OK) return st;
  if ((st = check_ranks(n_experts, n_ranks)) != MOE_OK) return st;
  if ((st = check_rows(hidden_dim, bytes_per_element)) != MOE_OK) return st;
  if (coselect && (coselect_tokens < 0 || coselect_tokens > tokens)) return MOE_EINVAL;
  if (!expert_counts || !rank_counts || !rank_offsets || !workspace || (dedup && !n_rows))
    return MOE_EINVAL;
  if (tokens > 0 && (!x || !topk_idx || !topk_gate || !send || !row_token || !row_experts ||
                     !row_weight || !slot_row || (dedup && !row_gates)))
    return MOE_EINVAL;
  const int d = dedup ? 1 : 0;
  if (workspace_bytes < moe_workspace_bytes(tokens, n_experts, top_k, n_ranks, d))
    return MOE_EWORKSPACE;
  const int rb = hidden_dim * bytes_per_element;
  const int64_t ncs = coselect ? coselect_tokens : 0;
  int32_t* eo = d ? nullptr : expert_offsets;
  hipStream_t s = as_stream(stream);
  if (moe::dispatch_scans_plan(tokens, n_experts, top_k, n_ranks, d, rb))
    return hip_status(moe::launch_dispatch_scan(
        x, topk_idx, topk_gate, tokens, rb, n_experts, top_k, n_ranks, placement, workspace, d,
        send, row_token, row_experts, d ? row_gates : nullptr, row_weight, slot_row,
        d ? n_rows : nullptr, expert_counts, rank_counts, rank_offsets, eo, ncs, coselect, s));
  // larger plans: the scan kernel, then the dispatch
  if (moe::launch_plan_scan(tokens, n_experts, top_k, n_ranks, placement, d, expert_counts,
                            rank_counts, rank_offsets, eo, workspace, s) != hipSuccess)
    return MOE_EHIP;
  if (tokens == 0 && !d) return MOE_OK;
  return hip_status(moe::launch_dispatch(x, topk_idx, topk_gate, tokens, rb, n_experts, top_k,
                                         n_ranks, workspace, d, send, row_token, row_experts,
                                         d ? row_gates : nullptr, row_weight, slot_row,
                                         d ? n_rows : nullptr, ncs, coselect, s));
}

// Rows of bf16 (2 bytes) or fp8 E4M3 (1 byte); the output is bf16.
static int check_combine(int64_t tokens, int hidden_dim, int top_k, int bytes_per_element) {
  if (tokens < 0 || top_k < 1 || hidden_dim < 1 || bytes_per_element < 1) return MOE_EINVAL;
  if (top_k > MOE_MAX_TOP_K || (bytes_per_element != 2 && bytes_per_element != 1))
    return MOE_EUNSUPPORTED;
  if (tokens > int64_t(INT_MAX) / top_k) return MOE_EUNSUPPORTED;
  const int64_t rb = int64_t(hidden_dim) * bytes_per_element;
  if (rb % 16 != 0 || int64_t(hidden_dim) * 2 > INT_MAX / 2) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

MOE_API int moe_combine(const void* rows, const float* row_weight, const int32_t* slot_row,
                        int64_t tokens, int hidden_dim, int top_k, int bytes_per_element,
                        void* out, void* stream) {
  const int st = check_combine(tokens, hidden_dim, top_k, bytes_per_element);
  if (st != MOE_OK) return st;
  if (tokens == 0) return MOE_OK;
  if (!rows || !slot_row || !out) return MOE_EINVAL;
  return hip_status(moe::launch_combine(rows, row_weight, slot_row, tokens,
                                        hidden_dim * bytes_per_element, top_k,
                                        bytes_per_element == 1, nullptr, out, as_stream(stream)));
}

MOE_API int moe_combine_route(const void* rows, const float* row_weight, const int32_t* slot_row,
                              int64_t tokens, int hidden_dim, int top_k, int bytes_per_element,
                              void* out, const float* next_logits, int64_t next_tokens,
                              int n_experts, int next_top_k, int gating, int n_ranks,
                              const int32_t* placement, int dedup, int32_t* next_topk_idx,
                              float* next_topk_gate, void* next_workspace,
                              size_t next_workspace_bytes, void* stream) {
  int st = check_combine(tokens, hidden_dim, top_k, bytes_per_element);
  if (st != MOE_OK) return st;
  if ((st = check_tek(next_tokens, n_experts, next_top_k)) != MOE_OK) return st;
  if ((st = check_ranks(n_experts, n_ranks)) != MOE_OK) return st;
  if (gating != 0 && gating != 1) return MOE_EINVAL;
  if (tokens > 0 && (!rows || !slot_row || !out)) return MOE_EINVAL;
  if (!next_workspace ||
      (next_tokens > 0 && (!next_logits || !next_topk_idx || !next_topk_gate)))
    return MOE_EINVAL;
  const int d = dedup ? 1 : 0;
  if (next_workspace_bytes < moe_workspace_bytes(next_tokens, n_experts, next_top_k, n_ranks, d))
    return MOE_EWORKSPACE;
  return hip_status(moe::launch_combine_route(
      rows, row_weight, slot_row, tokens, hidden_dim * bytes_per_element, top_k,
      bytes_per_element == 1, out, next_logits, next_tokens, n_experts, next_top_k, gating,
      n_ranks, placement, d, next_topk_idx, next_topk_gate, next_workspace, as_stream(stream)));
}

MOE_API size_t moe_expand_workspace_bytes(int64_t capacity, int n_experts, int top_k,
                                          int n_ranks) {
  if (check_tek(capacity, n_experts, top_k) != MOE_OK) return 0;
  if (check_ranks(n_experts, n_ranks) != MOE_OK) return 0;
  // the plan of the plain layout without its last region, the tile expert
  // bitmaps (only the co-selection counts of the routing call read them)
  return moe::plan_layout(capacity, n_experts, top_k, n_ranks, 0).bm_off;
}

MOE_API int moe_expand_counts(const int32_t* row_experts, const int32_t* n_rows,
                              int64_t capacity, int n_experts, int top_k, int n_ranks,
                              const int32_t* placement, int32_t* expert_counts,
                              int32_t* rank_counts, int32_t* rank_offsets,
                              int32_t* expert_offsets, void* workspace, size_t workspace_bytes,
                              void* stream) {
  int st = check_tek(capacity, n_experts, top_k);
  if (st != MOE_OK) return st;
  if ((st = check_ranks(n_experts, n_ranks)) != MOE_OK) return st;
  if ((capacity > 0 && !row_experts) || !n_rows || !expert_counts || !rank_counts ||
      !rank_offsets || !workspace)
    return MOE_EINVAL;
  if (workspace_bytes < moe_expand_workspace_bytes(capacity, n_experts, top_k, n_ranks))
    return MOE_EWORKSPACE;
  return hip_status(moe::launch_expand_counts(row_experts, capacity, n_experts, top_k, n_ranks,
                                              placement, n_rows, expert_counts, rank_counts,
                                              rank_offsets, expert_offsets, workspace,
                                              as_stream(stream)));
}

MOE_API int moe_expand_permute(const void* rows, const float* row_gates, const int32_t* n_rows,
                               int64_t capacity, int hidden_dim, int n_experts, int top_k,
                               int n_ranks, int bytes_per_element, const void* workspace,
                               size_t workspace_bytes, void* expanded, int64_t expanded_capacity,
                               int32_t* exp_row, int32_t* exp_expert, float* exp_gate,
                               int32_t* row_slot, void* stream) {
  int st = check_tek(capacity, n_experts, top_k);
  if (st != MOE_OK) return st;
  if ((st = check_ranks(n_experts, n_ranks)) != MOE_OK) return st;
  if ((st = check_rows(hidden_dim, bytes_per_element)) != MOE_OK) return st;
  if (expanded_capacity < 0 || !n_rows || !workspace) return MOE_EINVAL;
  if (expanded_capacity > int64_t(INT_MAX)) return MOE_EUNSUPPORTED;
  if (workspace_bytes < moe_expand_workspace_bytes(capacity, n_experts, top_k, n_ranks))
    return MOE_EWORKSPACE;
  if (capacity == 0) return MOE_OK;
  if (!rows || !row_gates || !row_slot ||
      (expanded_capacity > 0 && (!expanded || !exp_row || !exp_expert || !exp_gate)))
    return MOE_EINVAL;
  return hip_status(moe::launch_expand(rows, row_gates, n_rows, capacity,
                                       hidden_dim * bytes_per_element, n_experts, top_k, n_ranks,
                                       workspace, expanded, expanded_capacity, exp_row,
                                       exp_expert, exp_gate, row_slot, as_stream(stream)));
}

MOE_API int moe_expand_reduce(const void* expert_out, const float* exp_gate,
                              const int32_t* row_slot, const int32_t* n_rows, int64_t capacity,
                              int hidden_dim, int top_k, int bytes_per_element, void* out,
                              void* stream) {
  const int st = check_combine(capacity, hidden_dim, top_k, bytes_per_element);
  if (st != MOE_OK) return st;
  if (!n_rows) return MOE_EINVAL;
  if (capacity == 0) return MOE_OK;
  if (!expert_out || !row_slot || !out) return MOE_EINVAL;
  return hip_status(moe::launch_combine(expert_out, exp_gate, row_slot, capacity,
                                        hidden_dim * bytes_per_element, top_k,
                                        bytes_per_element == 1, n_rows, out, as_stream(stream)));
}

MOE_API int moe_coselect_counts(const int32_t* topk_idx, int64_t tokens, int n_experts,
                                int top_k, int32_t* coselect, void* stream) {
  int st = check_tek(tokens, n_experts, top_k);
  if (st != MOE_OK) return st;
  if (tokens == 0) return MOE_OK;
  if (!topk_idx || !coselect) return MOE_EINVAL;
  return hip_status(moe::launch_coselect(topk_idx, tokens, n_experts, top_k, coselect,
                                         as_stream(stream)));
}

MOE_API int moe_placement_search(const int32_t* coselect, int n_experts, int n_ranks,
                                 const int32_t* initial, int max_swaps, int32_t* placement,
                                 int64_t* objective, int* swaps) {
  if (n_experts < 1) return MOE_EINVAL;
  if (n_experts > MOE_MAX_EXPERTS) return MOE_EUNSUPPORTED;
  int st = check_ranks(n_experts, n_ranks);
  if (st != MOE_OK) return st;
  if (!coselect || !placement || max_swaps < 0) return MOE_EINVAL;
  if (initial) {
    int per[MOE_MAX_RANKS] = {0};
    for (int e = 0; e < n_experts; ++e) {
      if (initial[e] < 0 || initial[e] >= n_ranks) return MOE_EINVAL;
      ++per[initial[e]];
    }
    for (int r = 0; r < n_ranks; ++r)
      if (per[r] != n_experts / n_ranks) return MOE_EINVAL;
  }
  try {
    return moe::placement_search(coselect, n_experts, n_ranks, initial, max_swaps, placement,
                                 objective, swaps);
  } catch (...) {  // its host tables could not be allocated; no exception leaves the ABI
    return MOE_EUNSUPPORTED;
  }
}

MOE_API int moe_shuffle_fit(const int32_t* prev_idx, const int32_t* cur_idx,
                            const int32_t* next_idx, int64_t tokens, int n_experts, int top_k,
                            int n_ranks, const int32_t* placement_next, int32_t* pair_counts,
                            int32_t* single_counts, void* stream) {
  int st = check_tek(tokens, n_experts, top_k);
  if (st != MOE_OK) return st;
  if ((st = check_ranks(n_experts, n_ranks)) != MOE_OK) return st;
  if (!pair_counts || !single_counts) return MOE_EINVAL;
  if (tokens == 0) return MOE_OK;
  if (!prev_idx || !cur_idx || !next_idx) return MOE_EINVAL;
  return hip_status(moe::launch_shuffle_fit(prev_idx, cur_idx, next_idx, tokens, n_experts, top_k,
                                            n_ranks, placement_next, pair_counts, single_counts,
                                            as_stream(stream)));
}

MOE_API int moe_shuffle_predict(const int32_t* prev_idx, const int32_t* cur_idx, int64_t tokens,
                                int n_experts, int top_k, int n_ranks, const int32_t* pair_counts,
                                const int32_t* single_counts, int min_obs, float* scores,
                                void* stream) {
  int st = check_tek(tokens, n_experts, top_k);
  if (st != MOE_OK) return st;
  if ((st = check_ranks(n_experts, n_ranks)) != MOE_OK) return st;
  if (min_obs < 0) return MOE_EINVAL;
  if (tokens > int64_t(INT_MAX) / n_ranks) return MOE_EUNSUPPORTED;
  if (tokens == 0) return MOE_OK;
  if (!prev_idx || !cur_idx || !pair_counts || !single_counts || !scores) return MOE_EINVAL;
  return hip_status(moe::launch_shuffle_predict(prev_idx, cur_idx, tokens, n_experts, top_k,
                                                n_ranks, pair_counts, single_counts, min_obs,
                                                scores, as_stream(stream)));
}

MOE_API int moe_shuffle_assign(const float* scores, int64_t tokens, int n_ranks, int32_t* owner) {
  if (tokens < 0 || n_ranks < 1) return MOE_EINVAL;
  if (n_ranks > MOE_MAX_RANKS) return MOE_EUNSUPPORTED;
  if (tokens % n_ranks != 0) return MOE_EINVAL;
  if (tokens == 0) return MOE_OK;
  if (!scores || !owner) return MOE_EINVAL;
  try {
    return moe::shuffle_assign(scores, tokens, n_ranks, owner);
  } catch (...) {  // its host tables (16 bytes per token) could not be allocated
    return MOE_EUNSUPPORTED;
  }
}
