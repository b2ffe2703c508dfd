/*
 * The C ABI used from plain C (C11, no torch, no C++): one step of the path on
 * synthetic inputs - moe_route_plan, moe_dispatch_permute, moe_combine - with
 * device buffers from hipMalloc, then checks that follow from the definitions
 * alone:
 *   - rank_offsets is the exclusive scan of rank_counts and ends at T*k, and
 *     expert_counts sums to T*k (one row per token-expert assignment);
 *   - every send row is bit-equal to x[row_token] and every slot points at a
 *     row of its own token;
 *   - identity experts with gates summing to 1: combine returns x exactly;
 *   - the co-selection diagonal sums to T*k.
 * Then the same batch three times through the pipelined loop over two buffer
 * sets - moe_combine_route with no rows routes the first batch, then per
 * batch moe_dispatch_routed and a moe_combine_route that combines it and
 * routes the next into the other set - and checks that every dispatch gives
 * the rows and slots of the one-call step above and every combine returns x.
 * Prints "abi_demo ok" and exits 0, or names the first failed check and exits 1.
 * Built by the package build (gcc, linked against libmoe_route.so).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe_route.h"

#define T 1000
#define H 256
#define E 64
#define K 6
#define R 16

#define CHECK_HIP(call)                                                     \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                 \
      printf("abi_demo: %s failed: %s\n", #call, hipGetErrorString(e_));    \
      return 1;                                                             \
    }                                                                       \
  } while (0)

#define CHECK_MOE(call)                                                     \
  do {                                                                      \
    int s_ = (call);                                                        \
    if (s_ != MOE_OK) {                                                     \
      printf("abi_demo: %s failed: %s\n", #call, moe_status_string(s_));    \
      return 1;                                                             \
    }                                                                       \
  } while (0)

#define REQUIRE(cond, what)                                                 \
  do {                                                                      \
    if (!(cond)) {                                                          \
      printf("abi_demo: check failed: %s\n", what);                         \
      return 1;                                                             \
    }                                                                       \
  } while (0)

/* xorshift64*: the demo's own deterministic inputs */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 0x2545F4914F6CDD1Dull;
}

int main(void) {
  static float logits[T * E];
  static uint16_t x[T * H], send[T * K * H], out[T * H];
  static int32_t row_token[T * K], slot_row[T * K], W[E * E];
  int32_t expert_counts[E], rank_counts[R], rank_offsets[R + 1], expert_offsets[E];
  for (int i = 0; i < T * E; ++i)
    logits[i] = (float)((int64_t)(next_u64() >> 40) - (1 << 23)) / (float)(1 << 22);
  for (int i = 0; i < T * H; ++i) {
    uint16_t b = (uint16_t)(next_u64() >> 48);
    if ((b & 0x7F80u) == 0x7F80u) b &= 0xBFFFu; /* no Inf / NaN */
    x[i] = b;
  }

  const size_t ws_bytes = moe_workspace_bytes(T, E, K, R, 0);
  REQUIRE(ws_bytes > 0, "moe_workspace_bytes");
  float *d_logits, *d_gate, *d_row_weight;
  void *d_x, *d_send, *d_out, *d_ws;
  int32_t *d_idx, *d_ec, *d_rc, *d_ro, *d_eo, *d_W, *d_row_token, *d_row_expert, *d_slot_row;
  CHECK_HIP(hipMalloc((void**)&d_logits, sizeof logits));
  CHECK_HIP(hipMalloc((void**)&d_gate, sizeof(float) * T * K));
  CHECK_HIP(hipMalloc((void**)&d_idx, sizeof(int32_t) * T * K));
  CHECK_HIP(hipMalloc((void**)&d_ec, sizeof expert_counts));
  CHECK_HIP(hipMalloc((void**)&d_rc, sizeof rank_counts));
  CHECK_HIP(hipMalloc((void**)&d_ro, sizeof rank_offsets));
  CHECK_HIP(hipMalloc((void**)&d_eo, sizeof expert_offsets));
  CHECK_HIP(hipMalloc((void**)&d_W, sizeof W));
  CHECK_HIP(hipMalloc(&d_ws, ws_bytes));
  CHECK_HIP(hipMalloc(&d_x, sizeof x));
  CHECK_HIP(hipMalloc(&d_send, sizeof send));
  CHECK_HIP(hipMalloc(&d_out, sizeof out));
  CHECK_HIP(hipMalloc((void**)&d_row_token, sizeof row_token));
  CHECK_HIP(hipMalloc((void**)&d_row_expert, sizeof(int32_t) * T * K));
  CHECK_HIP(hipMalloc((void**)&d_row_weight, sizeof(float) * T * K));
  CHECK_HIP(hipMalloc((void**)&d_slot_row, sizeof slot_row));
  CHECK_HIP(hipMemcpy(d_logits, logits, sizeof logits, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_x, x, sizeof x, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemset(d_W, 0, sizeof W));

  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  CHECK_MOE(moe_route_plan(d_logits, T, E, K, 0, R, NULL, 0, d_idx, d_gate, d_ec, d_rc, d_ro,
                           d_eo, 0, NULL, d_ws, ws_bytes, stream));
  /* the co-selection counts of all T tokens, in the dispatch launch */
  CHECK_MOE(moe_dispatch_permute(d_x, d_idx, d_gate, T, H, E, K, R, 2, d_ws, ws_bytes,
                                 d_send, d_row_token, d_row_expert, d_row_weight, d_slot_row,
                                 T, d_W, stream));
  CHECK_MOE(moe_combine(d_send, d_row_weight, d_slot_row, T, H, K, 2, d_out, stream));
  CHECK_HIP(hipStreamSynchronize(stream));

  CHECK_HIP(hipMemcpy(expert_counts, d_ec, sizeof expert_counts, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(rank_counts, d_rc, sizeof rank_counts, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(rank_offsets, d_ro, sizeof rank_offsets, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(send, d_send, sizeof send, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(row_token, d_row_token, sizeof row_token, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(slot_row, d_slot_row, sizeof slot_row, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(W, d_W, sizeof W, hipMemcpyDeviceToHost));

  int64_t sum = 0;
  for (int e = 0; e < E; ++e) sum += expert_counts[e];
  REQUIRE(sum == (int64_t)T * K, "expert counts sum to T*k");
  REQUIRE(rank_offsets[0] == 0, "first offset is 0");
  for (int r = 0; r < R; ++r)
    REQUIRE(rank_offsets[r + 1] - rank_offsets[r] == rank_counts[r], "offsets scan the counts");
  REQUIRE(rank_offsets[R] == T * K, "offsets end at T*k");
  for (int p = 0; p < T * K; ++p) {
    REQUIRE(row_token[p] >= 0 && row_token[p] < T, "row token in range");
    REQUIRE(memcmp(send + (size_t)p * H, x + (size_t)row_token[p] * H, H * 2) == 0,
            "send row equals x[row_token]");
  }
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < K; ++j) {
      const int p = slot_row[t * K + j];
      REQUIRE(p >= 0 && p < T * K && row_token[p] == t, "slot points at a row of its token");
    }
  REQUIRE(memcmp(out, x, sizeof x) == 0, "identity experts: combine returns x");
  int64_t diag = 0;
  for (int e = 0; e < E; ++e) diag += W[e * E + e];
  REQUIRE(diag == (int64_t)T * K, "co-selection diagonal sums to T*k");

  /* the pipelined loop: set b % 2 holds batch b's ids, gates, plan, rows and
     output; batch b + 1 is routed into the other set by batch b's combine */
  enum { NB = 3 };
  float *p_gate[2], *p_row_weight[2];
  int32_t *p_idx[2], *p_row_token[2], *p_row_expert[2], *p_slot_row[2];
  void *p_ws[2], *p_send[2], *p_out[2];
  static uint16_t send2[T * K * H], out2[T * H];
  static int32_t slot_row2[T * K];
  for (int i = 0; i < 2; ++i) {
    CHECK_HIP(hipMalloc((void**)&p_gate[i], sizeof(float) * T * K));
    CHECK_HIP(hipMalloc((void**)&p_row_weight[i], sizeof(float) * T * K));
    CHECK_HIP(hipMalloc((void**)&p_idx[i], sizeof(int32_t) * T * K));
    CHECK_HIP(hipMalloc((void**)&p_row_token[i], sizeof(int32_t) * T * K));
    CHECK_HIP(hipMalloc((void**)&p_row_expert[i], sizeof(int32_t) * T * K));
    CHECK_HIP(hipMalloc((void**)&p_slot_row[i], sizeof(int32_t) * T * K));
    CHECK_HIP(hipMalloc(&p_ws[i], ws_bytes));
    CHECK_HIP(hipMalloc(&p_send[i], sizeof send));
    CHECK_HIP(hipMalloc(&p_out[i], sizeof out));
  }
  CHECK_MOE(moe_combine_route(NULL, NULL, NULL, 0, H, K, 2, NULL, d_logits, T, E, K, 0, R, NULL,
                              0, p_idx[0], p_gate[0], p_ws[0], ws_bytes, stream));
  for (int b = 0; b < NB; ++b) {
    const int c = b % 2, n = 1 - c;
    const int64_t next_tokens = b + 1 < NB ? T : 0;
    CHECK_MOE(moe_dispatch_routed(d_x, p_idx[c], p_gate[c], T, H, E, K, R, NULL, 0, 2, d_ec,
                                  d_rc, d_ro, d_eo, p_send[c], p_row_token[c], p_row_expert[c],
                                  NULL, p_row_weight[c], p_slot_row[c], NULL, 0, NULL, p_ws[c],
                                  ws_bytes, stream));
    CHECK_MOE(moe_combine_route(p_send[c], p_row_weight[c], p_slot_row[c], T, H, K, 2, p_out[c],
                                d_logits, next_tokens, E, K, 0, R, NULL, 0, p_idx[n], p_gate[n],
                                p_ws[n], ws_bytes, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(send2, p_send[c], sizeof send2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(slot_row2, p_slot_row[c], sizeof slot_row2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(out2, p_out[c], sizeof out2, hipMemcpyDeviceToHost));
    REQUIRE(memcmp(send2, send, sizeof send) == 0, "pipelined rows equal the one-call rows");
    REQUIRE(memcmp(slot_row2, slot_row, sizeof slot_row) == 0,
            "pipelined slots equal the one-call slots");
    REQUIRE(memcmp(out2, x, sizeof x) == 0, "pipelined combine returns x");
  }
  for (int i = 0; i < 2; ++i) {
    hipFree(p_gate[i]); hipFree(p_row_weight[i]); hipFree(p_idx[i]); hipFree(p_row_token[i]);
    hipFree(p_row_expert[i]); hipFree(p_slot_row[i]); hipFree(p_ws[i]); hipFree(p_send[i]);
    hipFree(p_out[i]);
  }

  CHECK_HIP(hipStreamDestroy(stream));
  hipFree(d_logits); hipFree(d_gate); hipFree(d_idx); hipFree(d_ec); hipFree(d_rc);
  hipFree(d_ro); hipFree(d_eo); hipFree(d_W); hipFree(d_ws); hipFree(d_x); hipFree(d_send);
  hipFree(d_out); hipFree(d_row_token); hipFree(d_row_expert); hipFree(d_row_weight);
  hipFree(d_slot_row);
  printf("abi_demo ok: T=%d H=%d E=%d k=%d R=%d, one-call step and %d pipelined batches\n", T, H,
         E, K, R, NB);
  return 0;
}
