/*
 * moe_route.h - per-GPU MoE expert-parallel dispatch and combine on AMD
 * Instinct MI355X (gfx950).  Plain C ABI over hand-written HIP kernels.
 *
 * What is computed (page title, then section):
 *  [EC] "Expert Coupling in MoE Pretraining: Reducing All-to-All Overhead with
 *       Correlated Placement and Token Shuffling" (summary page):
 *       "Background" (top-k routing), "The Communication Bottleneck" (dispatch,
 *       experts, combine under expert parallelism), "Method 1: Correlated Expert
 *       Placement + Deduplicating Dispatcher" (one row per (token, expert) vs one
 *       row per distinct (token, destination rank) with expert ids and routing
 *       probabilities; co-selection graph W; E/EP experts per GPU).
 *  [DD] "DODOCO: MoE AlltoAll Traffic Matrices on Real Text" (dataset card):
 *       "Setup" (contiguous placement; per-destination input splits),
 *       "Reading the counts" (one count per token-expert assignment, rows sum to
 *       tokens x top-k, payload = count x hidden x bytes per element, expert
 *       block sums = receive totals), "send_matrices.csv columns" (combine moves
 *       the same volumes back).
 *  [AD] "AllToAllDispatchScenario" (mlsysim API page), "Attributes": the
 *       problem's inputs are the token count, device count, expert count, hidden
 *       size and bytes per element; the argument names below follow them
 *       (tokens, n_ranks, n_experts, hidden_dim, bytes_per_element).
 *
 * Destination ranks are logical: rank r's rows are the contiguous segment
 * [rank_offsets[r], rank_offsets[r+1]) of one send buffer on this GPU.
 *
 * Conventions shared by every entry point
 *  - Every pointer argument is DEVICE memory (hipMalloc'd or a torch tensor's
 *    data pointer) unless it is marked "host".  All buffers are caller-owned;
 *    the library allocates nothing, keeps no state between calls and frees
 *    nothing.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *    is enqueued asynchronously on it; the call returns once the launches are
 *    queued.  Calls on one stream execute in order.
 *  - Arrays are dense, row-major, with no padding: [T][k] means element (t, j)
 *    is at t*k + j.  T = tokens, E = n_experts, k = top_k, R = n_ranks,
 *    H = hidden_dim, N = T*k.
 *  - Return value: MOE_OK, or an error code.  Argument checks run on the host
 *    before anything is enqueued, so on an error nothing has been launched and
 *    no output has been touched.  MOE_EHIP means a launch failed (outputs are
 *    then undefined).  No C++ exception crosses the ABI.
 *  - tokens == 0 is valid: nothing is launched except what is documented.
 *  - Limits: 1 <= k <= 16, k <= E <= 1024, 1 <= R <= 64, E % R == 0,
 *    T*k < 2^31.  Outside them: MOE_EUNSUPPORTED (or MOE_EINVAL for values
 *    that can never be valid).
 *  - Device-side contents are preconditions that the host cannot check without
 *    synchronising: expert ids in topk_idx must lie in [0, E) and placement
 *    values in [0, R).  Out-of-range values are clamped inside the kernels so
 *    that no access leaves its buffer; the results are then unspecified.
 *  - Concurrent calls are safe when they use distinct output and workspace
 *    buffers.
 */
#ifndef MOE_ROUTE_H_
#define MOE_ROUTE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_EINVAL 1        /* an argument can never be valid (null pointer, k > E, ...) */
#define MOE_EUNSUPPORTED 2  /* valid for the method but outside this library's limits */
#define MOE_EWORKSPACE 3    /* workspace_bytes is smaller than moe_workspace_bytes() */
#define MOE_EHIP 4          /* a HIP launch failed */

#define MOE_MAX_TOP_K 16
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_RANKS 64

/* Host.  A static, NUL-terminated description of a status code (never NULL). */
const char* moe_status_string(int status);

/* Host.  Bytes of workspace that moe_send_counts() or moe_route_plan() fills
 * and the dispatch call of the same topk_idx and dedup mode then reads.
 * Returns 0 if the arguments are outside the limits above.  The workspace is
 * opaque; it needs no initialisation and 256-byte alignment is enough. */
size_t moe_workspace_bytes(int64_t tokens, int n_experts, int top_k, int n_ranks, int dedup);

/* A1 - top-k routing ([EC] "Background"): each token is routed to its k experts
 * with the largest router logits.
 *   logits     [T][E] fp32, read only.
 *   topk_idx   [T][k] int32 out: the selected expert ids in order of logit,
 *              largest first; equal logits (IEEE equality, so -0.0 == +0.0) go
 *              to the lower expert id first.  NaN logits are not supported.
 *   topk_gate  [T][k] fp32 out: softmax over the k selected logits,
 *              g_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), evaluated in fp64 and
 *              rounded once to fp32 (the pages name "routing probabilities" but
 *              not their formula; this is the plainest reading).
 * Errors: MOE_EINVAL for null pointers, tokens < 0, E < 1, k < 1, k > E. */
int moe_route_topk(const float* logits, int64_t tokens, int n_experts, int top_k,
                   int32_t* topk_idx, float* topk_gate, void* stream);

/* A1, gating variant: the same expert selection as moe_route_topk(), with
 * topk_gate[t][j] = exp(l_j - l_0) / (sum over all E experts e of
 * exp(l_e - l_0)), i.e. the softmax over every expert's logit taken at the
 * selected ones, not renormalised over the selection (the pages speak of
 * routing probabilities without fixing the normalisation; this is the other
 * common reading).  fp64 inside, one rounding to fp32.  Arguments and errors
 * as moe_route_topk(). */
int moe_route_topk_softmax_all(const float* logits, int64_t tokens, int n_experts, int top_k,
                               int32_t* topk_idx, float* topk_gate, void* stream);

/* A2 + A3 - send counts and their exclusive scan ([DD] "Setup", "Reading the
 * counts"; [EC] "Method 1").
 *   topk_idx       [T][k] int32, read only (expert ids in [0, E)).
 *   placement      [E] int32 expert -> rank, values in [0, R), read only; NULL
 *                  means contiguous: rank r holds experts r*E/R .. (r+1)*E/R-1.
 *                  The pages' placements hold exactly E/R experts per rank; the
 *                  kernels do not need that property.
 *   dedup          0: one row per (token, expert) - rank_counts[r] counts the
 *                  token-expert assignments whose expert lives on r (each row of
 *                  the send matrix sums to T*k).  1: one row per distinct (token,
 *                  rank) - rank_counts[r] counts the tokens with at least one
 *                  selected expert on r.
 *   expert_counts  [E] int32 out: #(t, j) with topk_idx[t][j] == e (both modes).
 *   rank_counts    [R] int32 out, as above.
 *   rank_offsets   [R+1] int32 out: exclusive scan of rank_counts; rank r's rows
 *                  are [rank_offsets[r], rank_offsets[r+1]); rank_offsets[R] is
 *                  the total number of rows (N, or D in dedup mode).
 *   expert_offsets [E] int32 out, may be NULL; written only when dedup == 0:
 *                  the first row of expert e's segment.  Inside a rank, experts
 *                  are laid out in ascending id.
 *   workspace      device buffer of at least moe_workspace_bytes(...) bytes; it
 *                  receives the per-tile plan that the dispatch call consumes.
 * Errors: MOE_EINVAL (null required pointer, bad sizes, E % R != 0),
 *         MOE_EUNSUPPORTED (limits), MOE_EWORKSPACE. */
int moe_send_counts(const int32_t* topk_idx, int64_t tokens, int n_experts, int top_k,
                    int n_ranks, const int32_t* placement, int dedup,
                    int32_t* expert_counts, int32_t* rank_counts, int32_t* rank_offsets,
                    int32_t* expert_offsets, void* workspace, size_t workspace_bytes,
                    void* stream);

/* A1 + A2 + A3 (+ A6) in one call: moe_route_topk() (gating 0) or
 * moe_route_topk_softmax_all() (gating 1), then moe_send_counts() on the ids
 * it produced, then (coselect_tokens > 0) moe_coselect_counts() on the first
 * coselect_tokens of them - the same outputs bit for bit and the same plan left
 * in the workspace ([EC] "Background", "Method 1", "Correlation Formation and
 * Stability"; [DD] "Setup", "Reading the counts").  For E <= 256 one kernel
 * routes each 32-token tile and counts it (one workgroup per tile), which saves
 * the counting kernel's launch and its reread of topk_idx; larger E (or
 * T > 2^24) run the separate kernels.  Co-selection counts, when asked for,
 * come from the expert bitmaps the plan keeps, in one more short launch (the
 * dispatch calls can take them in their own launch instead).
 *   logits, topk_idx, topk_gate   as moe_route_topk() (may be NULL when
 *                                 tokens == 0).
 *   gating                        0 or 1, as above.
 *   n_ranks ... expert_offsets    as moe_send_counts().
 *   coselect_tokens               0 <= coselect_tokens <= tokens; 0: no
 *                                 co-selection counts.
 *   coselect                      [E][E] int32, ACCUMULATED as by
 *                                 moe_coselect_counts(); may be NULL when
 *                                 coselect_tokens == 0.
 *   workspace, workspace_bytes    as moe_send_counts().
 * Errors: those of moe_route_topk() and moe_send_counts(); MOE_EINVAL for a
 *         gating value other than 0 or 1 or a bad coselect_tokens. */
int moe_route_plan(const float* logits, int64_t tokens, int n_experts, int top_k, int gating,
                   int n_ranks, const int32_t* placement, int dedup, int32_t* topk_idx,
                   float* topk_gate, int32_t* expert_counts, int32_t* rank_counts,
                   int32_t* rank_offsets, int32_t* expert_offsets, int64_t coselect_tokens,
                   int32_t* coselect, void* workspace, size_t workspace_bytes, void* stream);

/* A4a - dispatch permute, one row per (token, expert) ([EC] "Method 1",
 * conventional dispatch; [DD] "Reading the counts").
 * Must follow moe_send_counts(dedup = 0), or moe_route_plan(dedup = 0), on the
 * same stream with the same topk_idx and workspace.  The workspace carries the
 * plan: every row position, and with it the placement and the expert and rank
 * offsets of the counts call, so the dispatch calls take none of them.
 *   x            [T][H] elements of bytes_per_element bytes (bf16: 2), read only;
 *                rows are copied bit for bit.  H * bytes_per_element must be a
 *                multiple of 16.
 *   topk_gate    [T][k] fp32, read only.
 *   send         [N][H] out.  Row order: rank ascending; inside a rank, expert id
 *                ascending; inside an expert, token ascending.
 *   row_token    [N] int32 out: source token of each row.
 *   row_expert   [N] int32 out: expert of each row.
 *   row_weight   [N] fp32 out: the gate of that (token, expert).
 *   slot_row     [T][k] int32 out: the row that carries slot j of token t.
 *   coselect     [E][E] int32 or NULL.  Non-NULL: the co-selection counts of
 *                the first coselect_tokens tokens (0 <= coselect_tokens <=
 *                tokens) are ADDED to it exactly as moe_coselect_counts() would
 *                add them (A6, [EC] "Method 1"), in the same launch as the row
 *                copies: the plan holds every token's expert bitmaps.  NULL:
 *                coselect_tokens is ignored.  The matrix must not alias an
 *                output and must not be updated concurrently by another call.
 * Errors: MOE_EINVAL (also coselect_tokens outside [0, tokens] with coselect
 *         non-NULL), MOE_EUNSUPPORTED (bytes_per_element not 1/2/4, row bytes
 *         not a multiple of 16, limits), MOE_EWORKSPACE. */
int moe_dispatch_permute(const void* x, const int32_t* topk_idx, const float* topk_gate,
                         int64_t tokens, int hidden_dim, int n_experts, int top_k,
                         int n_ranks, int bytes_per_element, const void* workspace,
                         size_t workspace_bytes, void* send, int32_t* row_token,
                         int32_t* row_expert, float* row_weight, int32_t* slot_row,
                         int64_t coselect_tokens, int32_t* coselect, void* stream);

/* Bytes of the per-device scratch array of moe_dispatch_permute_noalloc(). */
#define MOE_NOALLOC_SCRATCH_BYTES (8u << 20)

/* A2 + A3 + A4a without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, serving loops and harnesses that
 * forbid hipMalloc.  The same as moe_send_counts(dedup = 0) followed by
 * moe_dispatch_permute() on the same stream - the same outputs, bit for bit -
 * except that the plan goes to a static scratch array of the library instead
 * of a caller workspace: MOE_NOALLOC_SCRATCH_BYTES (8 MiB) of device memory
 * that every GPU the library runs on holds from this call's first use on it
 * until the process ends.  Nothing is allocated: no hipMalloc, hipFree or
 * allocating library routine is called.
 *   Arguments: those of moe_send_counts() (placement, the counts and offsets,
 *   expert_offsets may be NULL) and moe_dispatch_permute() (x .. slot_row; no
 *   co-selection counts).
 *   Every call on one GPU uses that GPU's one scratch array, which keeps the
 *   last call's plan (nothing in it needs to start at zero): calls that can
 *   overlap in time on one GPU - on streams not ordered with each other, or
 *   from several host threads - race on it and must not be made.
 * Errors: those of moe_send_counts() and moe_dispatch_permute();
 *   MOE_EUNSUPPORTED when the plan, moe_workspace_bytes(tokens, n_experts,
 *   top_k, n_ranks, 0) bytes, exceeds MOE_NOALLOC_SCRATCH_BYTES (about 35
 *   bytes per token at 64 experts, top-6: some 240,000 tokens); MOE_EHIP when
 *   the scratch's device address cannot be obtained or a launch fails. */
int moe_dispatch_permute_noalloc(const void* x, const int32_t* topk_idx, const float* topk_gate,
                                 int64_t tokens, int hidden_dim, int n_experts, int top_k,
                                 int n_ranks, const int32_t* placement, int bytes_per_element,
                                 int32_t* expert_counts, int32_t* rank_counts,
                                 int32_t* rank_offsets, int32_t* expert_offsets, void* send,
                                 int32_t* row_token, int32_t* row_expert, float* row_weight,
                                 int32_t* slot_row, void* stream);

/* A4b - deduplicating dispatch, one row per distinct (token, destination rank)
 * ([EC] "Method 1", deduplicating dispatcher).
 * Must follow moe_send_counts(dedup = 1), or moe_route_plan(dedup = 1), on the
 * same stream with the same topk_idx and workspace (which carries the plan,
 * the placement included).  Capacity is
 * N = T*k rows for every output so that no host synchronisation is needed; the
 * number of rows written, D, is stored in *n_rows (and equals rank_offsets[R]
 * of the counts call).
 *   send         [capacity N][H] out; rows [0, D) written.  Row order: rank
 *                ascending; inside a rank, token ascending.
 *   row_token    [N] int32 out.
 *   row_experts  [N][k] int32 out: the ids of the token's selected experts that
 *                live on the row's rank, ascending, padded with -1.
 *   row_gates    [N][k] fp32 out: their gates, aligned with row_experts, padded
 *                with 0.
 *   row_weight   [N] fp32 out: the sum of those gates (fp64, ascending expert
 *                order, rounded once), i.e. the combine weight of the row when
 *                the experts return their inputs unchanged.
 *   slot_row     [T][k] int32 out: the row that carries slot j of token t
 *                (slots whose experts share a rank share a row).
 *   n_rows       [1] int32 out: D.
 *   coselect_tokens, coselect: as moe_dispatch_permute().
 * Errors: as moe_dispatch_permute. */
int moe_dispatch_permute_dedup(const void* x, const int32_t* topk_idx, const float* topk_gate,
                               int64_t tokens, int hidden_dim, int n_experts, int top_k,
                               int n_ranks, int bytes_per_element, const void* workspace,
                               size_t workspace_bytes, void* send, int32_t* row_token,
                               int32_t* row_experts, float* row_gates, float* row_weight,
                               int32_t* slot_row, int32_t* n_rows, int64_t coselect_tokens,
                               int32_t* coselect, void* stream);

/* A1 + A2 + A3 + A4 (+ A6) - the whole send side in one call: the same as
 * moe_route_plan() (coselect_tokens 0) followed by moe_dispatch_permute()
 * (dedup = 0) or moe_dispatch_permute_dedup() (dedup = 1) on the same stream,
 * with the same outputs bit for bit, and afterwards the same plan in the
 * workspace (so further dispatch calls on it may follow).  It takes two
 * launches instead of three or four - the routing kernel counts the tiles, and
 * the dispatch workgroups scan the plan themselves - when E <= 256 and the
 * plan's position columns (E, or R in dedup mode) have V <= 2048 vectors of 16
 * tile counts (V = columns x ceil(T / 512)) with V x W <= 4 Mi, W being the
 * dispatch's workgroups (ceil(T x ceil(row bytes / 4 KiB) / 4) for rows of at
 * least 4 KiB): e.g. T = 4096 with up to 256 experts, plain, or T = 16384 of
 * 8 KiB rows with up to 16 ranks, dedup.  Other plans take the routing call's
 * scan (one kernel; two past 16384 tokens).
 *   logits, gating                as moe_route_plan().
 *   x, hidden_dim, bytes_per_element   as moe_dispatch_permute().
 *   topk_idx, topk_gate           [T][k] out.
 *   expert_counts .. expert_offsets    as moe_route_plan() (expert_offsets may
 *                                 be NULL; dedup leaves it unwritten).
 *   send, row_token, row_weight, slot_row   as the dispatch calls.
 *   row_experts   dedup: [N][k] int32 out, as moe_dispatch_permute_dedup();
 *                 plain: [N] int32 out, the row_expert of moe_dispatch_permute().
 *   row_gates     dedup: [N][k] fp32 out; plain: ignored (may be NULL).
 *   n_rows        dedup: [1] int32 out; plain: ignored (may be NULL).
 *   coselect_tokens, coselect     as moe_dispatch_permute().
 *   workspace, workspace_bytes    moe_workspace_bytes(tokens, n_experts,
 *                                 top_k, n_ranks, dedup) bytes.
 * Errors: those of moe_route_plan() and the dispatch call. */
int moe_route_dispatch(const float* logits, const void* x, int64_t tokens, int hidden_dim,
                       int n_experts, int top_k, int gating, int n_ranks,
                       const int32_t* placement, int dedup, int bytes_per_element,
                       int32_t* topk_idx, float* topk_gate, int32_t* expert_counts,
                       int32_t* rank_counts, int32_t* rank_offsets, int32_t* expert_offsets,
                       void* send, int32_t* row_token, int32_t* row_experts, float* row_gates,
                       float* row_weight, int32_t* slot_row, int32_t* n_rows,
                       int64_t coselect_tokens, int32_t* coselect, void* workspace,
                       size_t workspace_bytes, void* stream);

/* A5 - combine ([EC] "The Communication Bottleneck"; [DD] "send_matrices.csv
 * columns": combine moves the dispatch volumes back): each token's output is the
 * weighted sum of the rows that served it.
 *   rows         [*][H] read only: the rows returned by the experts, in the
 *                send-buffer layout of the dispatch call; bf16 when
 *                bytes_per_element is 2, fp8 E4M3 (OCP: 1 sign, 4 exponent bits
 *                with bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN)
 *                when it is 1 ([DD] "Reading the counts": the payload is count x
 *                hidden x bytes per element of the dispatch precision).
 *   row_weight   [*] fp32 or NULL (= 1 for every row).
 *   slot_row     [T][k] int32: rows of each token; negative entries are skipped
 *                and a row listed by several slots is added once.
 *   out          [T][H] bf16 out: out[t][h] = bf16(sum over the token's distinct
 *                rows r of row_weight[r] * rows[r][h]).  The pages fix neither
 *                the order nor the precision of this sum; here it is, exactly:
 *                acc = -0.0f, then for the distinct rows in ascending row index
 *                acc = fmaf(row_weight[r], rows[r][h], acc) in fp32 (one
 *                rounding per step, nearest-even, subnormals kept), then one
 *                round-to-nearest-even of acc to bf16 (overflow to infinity).
 *                Every fp8 value is decoded exactly.  The result is a pure
 *                function of the inputs, bit for bit, for every finite or
 *                infinite input; an output that the rule makes NaN (a NaN in a
 *                row, inf - inf, 0 * inf) is some NaN whose sign and payload
 *                are not specified.
 * Errors: MOE_EINVAL, MOE_EUNSUPPORTED (bytes_per_element not 1 or 2, H *
 *         bytes_per_element not a multiple of 16, k > 16). */
int moe_combine(const void* rows, const float* row_weight, const int32_t* slot_row,
                int64_t tokens, int hidden_dim, int top_k, int bytes_per_element,
                void* out, void* stream);

/* A5 + A1/A2 - the combine of one batch and the routing of the next, for a loop
 * over independent batches (microbatches of one layer): the same as
 * moe_combine() on this batch, then the routing and the per-tile counting of
 * moe_route_dispatch() on the next batch without its scan and its dispatch,
 * in one launch (the next batch's routing workgroups run beside this batch's
 * combine; more than 256 experts or 16 Mi next tokens: three launches).  A
 * moe_dispatch_routed() call on the next batch then scans the plan and
 * dispatches it.  The first batch of a loop is routed by a call with tokens 0
 * (the routing kernel alone).
 *   rows .. out, tokens, hidden_dim, top_k, bytes_per_element
 *                 as moe_combine() (tokens 0: no combine).
 *   next_logits   [next_tokens][E] fp32, as moe_route_plan()'s logits.
 *   next_tokens, n_experts, next_top_k, gating, n_ranks, placement, dedup
 *                 the next batch's routing, as moe_route_plan().
 *   next_topk_idx, next_topk_gate   [next_tokens][next_top_k] out.  The ids
 *                 are those of moe_route_topk(); the gates too with gating 0,
 *                 and within 1 ulp of them with gating 1 (both within 1 ulp
 *                 of the softmax over all logits: the fp64 sum over the
 *                 logits runs in another order).
 *   next_workspace, next_workspace_bytes   the next batch's plan (tile
 *                 counts, slot codes, expert bitmaps; not yet scanned):
 *                 moe_workspace_bytes(next_tokens, n_experts, next_top_k,
 *                 n_ranks, dedup) bytes, handed to moe_dispatch_routed().
 * The two batches' buffers must not overlap.
 * Errors: those of moe_combine() and moe_route_plan(). */
int moe_combine_route(const void* rows, const float* row_weight, const int32_t* slot_row,
                      int64_t tokens, int hidden_dim, int top_k, int bytes_per_element,
                      void* out, const float* next_logits, int64_t next_tokens, int n_experts,
                      int next_top_k, int gating, int n_ranks, const int32_t* placement,
                      int dedup, int32_t* next_topk_idx, float* next_topk_gate,
                      void* next_workspace, size_t next_workspace_bytes, void* stream);

/* A3 + A4 (+ A6) - the dispatch of a batch routed by moe_combine_route(): the
 * plan's scan and the dispatch, with the same outputs as the second half of
 * moe_route_dispatch() (two launches become one when the dispatch
 * workgroups scan the plan themselves, under the same limits).  Every
 * argument as moe_route_dispatch(), with topk_idx and topk_gate read only;
 * tokens, n_experts, top_k, n_ranks, placement and dedup must be those of the
 * routing call, and workspace the one it wrote (anything else gives an
 * undefined plan).
 * Errors: those of moe_route_dispatch(). */
int moe_dispatch_routed(const void* x, const int32_t* topk_idx, const float* topk_gate,
                        int64_t tokens, int hidden_dim, int n_experts, int top_k, int n_ranks,
                        const int32_t* placement, int dedup, int bytes_per_element,
                        int32_t* expert_counts, int32_t* rank_counts, int32_t* rank_offsets,
                        int32_t* expert_offsets, void* send, int32_t* row_token,
                        int32_t* row_experts, float* row_gates, float* row_weight,
                        int32_t* slot_row, int32_t* n_rows, int64_t coselect_tokens,
                        int32_t* coselect, void* workspace, size_t workspace_bytes,
                        void* stream);

/* A6 - expert co-selection counts ([EC] "Method 1": the correlation graph
 * counts the tokens that select both experts; "Correlation Formation and
 * Stability": about 4096 tokens suffice to fit it).
 *   topk_idx     [T][k] int32; the first `tokens` rows are used.
 *   coselect     [E][E] int32, ACCUMULATED: for every used token, +1 at
 *                [a][b] for each ordered pair of distinct selected experts and
 *                +1 at [a][a] for each selected expert.  Zero it before the
 *                first call.  Calls that accumulate into the same matrix must
 *                not run concurrently.
 * Errors: MOE_EINVAL (null pointers, bad sizes), MOE_EUNSUPPORTED. */
int moe_coselect_counts(const int32_t* topk_idx, int64_t tokens, int n_experts, int top_k,
                        int32_t* coselect, void* stream);

/* ------------------------------------------------------------------------
 * Receive side of the deduplicating dispatcher ([EC] "Method 1": a dedup row
 * carries the ids and routing probabilities of every selected expert on its
 * destination rank, so the receiving rank hands the row to each of them and
 * weights their outputs by those probabilities).
 *
 * The received rows are laid out as moe_dispatch_permute_dedup() writes them:
 * rows [C][H], row_experts [C][k] (ids ascending, -1 = empty column),
 * row_gates [C][k], and a device row count *n_rows <= C, where C = `capacity`
 * (host).  Rows at or past *n_rows are ignored, whatever they hold.
 * Expansion writes, for every received row p and every listed expert e, one
 * copy of row p into an expanded buffer ordered by (rank of e, e, p): the
 * layout of the conventional dispatcher, one contiguous segment per expert
 * (the input of a grouped expert GEMM).  After the experts ran, the reduction
 * turns each received row back into one row: the gate-weighted sum of its
 * experts' outputs.
 * ------------------------------------------------------------------------ */

/* Host.  Bytes of workspace moe_expand_counts() fills and moe_expand_permute()
 * then reads, for `capacity` received rows.  0 outside the limits. */
size_t moe_expand_workspace_bytes(int64_t capacity, int n_experts, int top_k, int n_ranks);

/* Receive-side counts and the expansion plan.
 *   row_experts    [C][k] int32, as above (ids in [0, E) or negative = empty).
 *   n_rows         device int32[1]: the number of received rows (<= C).
 *   capacity       host: C, the rows the buffers hold.
 *   placement      [E] or NULL = contiguous (as moe_send_counts()).
 *   expert_counts  [E] out: rows listing each expert (the per-expert receive
 *                  counts).
 *   rank_counts    [R] out: sum of expert_counts over each rank's experts.
 *   rank_offsets   [R+1] out: exclusive scan; rank_offsets[R] = the number of
 *                  expanded rows.
 *   expert_offsets [E] out or NULL: first expanded row of each expert; experts
 *                  ordered by (rank, id).
 *   workspace      >= moe_expand_workspace_bytes(C, E, k, R) bytes.
 * Errors: as moe_send_counts(); n_rows must not be NULL. */
int moe_expand_counts(const int32_t* row_experts, const int32_t* n_rows, int64_t capacity,
                      int n_experts, int top_k, int n_ranks, const int32_t* placement,
                      int32_t* expert_counts, int32_t* rank_counts, int32_t* rank_offsets,
                      int32_t* expert_offsets, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Receive-side expansion: copies every listed (row, expert) into its place.
 * The row_experts table is not an argument: moe_expand_counts() read it, and
 * the plan it left in the workspace holds every entry's expert and position.
 *   rows           [C][H] elements of bytes_per_element bytes (copied bitwise).
 *   row_gates      [C][k] fp32, aligned with the row_experts table.
 *   workspace      as filled by moe_expand_counts() for the same arguments.
 *   expanded       [expanded_capacity][H] out: expanded row q = rows[exp_row[q]].
 *   exp_row, exp_expert [expanded_capacity] int32 out; exp_gate
 *                  [expanded_capacity] fp32 out: source row, expert and that
 *                  expert's gate of each expanded row.
 *   row_slot       [C][k] int32 out: expanded row of (row p, column c); -1 for
 *                  empty columns, for rows at or past *n_rows, and for entries
 *                  that would land at or past expanded_capacity (those are not
 *                  written; rank_offsets[R] from moe_expand_counts() tells the
 *                  caller how many rows the expansion needs).
 * Errors: MOE_EINVAL, MOE_EUNSUPPORTED (as moe_dispatch_permute()),
 *         MOE_EWORKSPACE. */
int moe_expand_permute(const void* rows, const float* row_gates, const int32_t* n_rows,
                       int64_t capacity, int hidden_dim, int n_experts, int top_k, int n_ranks,
                       int bytes_per_element, const void* workspace, size_t workspace_bytes,
                       void* expanded, int64_t expanded_capacity, int32_t* exp_row,
                       int32_t* exp_expert, float* exp_gate, int32_t* row_slot,
                       void* stream);

/* Receive-side reduction: for every received row p < *n_rows,
 * out[p][h] = bf16(sum over the distinct expanded rows q in row_slot[p][.]
 * (q >= 0) of exp_gate[q] * expert_out[q][h]), with the arithmetic of
 * moe_combine() (fp32 fused multiply-adds from -0.0 over the rows in ascending
 * index, one round-to-nearest-even).  exp_gate NULL = weight 1.  Rows
 * p >= *n_rows of out are not written.
 *   expert_out     [expanded rows][H] bf16 (bytes_per_element 2) or fp8 E4M3
 *                  (1): the experts' outputs in the expanded layout.
 *   out            [C][H] bf16.
 * Errors: as moe_combine(); n_rows must not be NULL. */
int moe_expand_reduce(const void* expert_out, const float* exp_gate, const int32_t* row_slot,
                      const int32_t* n_rows, int64_t capacity, int hidden_dim, int top_k,
                      int bytes_per_element, void* out, void* stream);

/* Host.  Correlated expert placement ([EC] "Method 1": a Kernighan-Lin-style
 * local search starts from the contiguous placement and swaps experts between
 * ranks to maximise the co-selection weight of the pairs that share a rank;
 * each rank keeps E/R experts).  The search itself is not printed on the page;
 * this is the plainest reading: repeatedly apply the swap of two experts on
 * different ranks with the largest gain in
 *   O = sum over ordered pairs x != y on one rank of coselect[x][y],
 * ties to the lowest (e, f) with e < f, until no swap gains or `max_swaps`
 * swaps were made.  Synchronous, host memory only, deterministic.
 *   coselect   host [E][E] int32: W, e.g. moe_coselect_counts() copied back.
 *   initial    host [E] int32 or NULL (= contiguous): the starting placement;
 *              every rank must hold exactly E/R experts.
 *   max_swaps  >= 0.
 *   placement  host [E] int32 out: the expert -> rank table found.
 *   objective  host int64 out or NULL: O of the result.
 *   swaps      host int out or NULL: swaps made.
 * Errors: MOE_EINVAL (null pointers, E % R != 0, max_swaps < 0, an initial
 *         placement with a value outside [0, R) or not E/R experts per rank),
 *         MOE_EUNSUPPORTED (E > 1024, R > 64, or its E x R host table could not
 *         be allocated). */
int moe_placement_search(const int32_t* coselect, int n_experts, int n_ranks,
                         const int32_t* initial, int max_swaps, int32_t* placement,
                         int64_t* objective, int* swaps);

/* ------------------------------------------------------------------------
 * Token-shuffle planner ([EC] "Method 2: Token Shuffling").  Reading: the
 * rank that will serve a token at layer l+1 is guessed from its experts at
 * layers l-1 and l - from the pair, or from the layer-l expert alone when the
 * pair is rare in the calibration data - and the ranks then take equal shares
 * of the tokens, the surest guesses first.  No formula is printed; the
 * readings are stated per call.  The fused reduce-scatter that moves the
 * tokens is not part of this library.
 * ------------------------------------------------------------------------ */

/* Fit, on a calibration batch: for every token, every expert c it selects at
 * layer l+1 (on rank r = placement_next[c], contiguous when NULL) and every
 * pair (a, b) of its experts at layers l-1 (prev_idx) and l (cur_idx):
 *   pair_counts[a][b][r] += 1;  and for every b:  single_counts[b][r] += 1.
 *   prev_idx, cur_idx, next_idx  [T][k] int32 (ids in [0, E)).
 *   pair_counts    [E][E][R] int32, ACCUMULATED (zero it first).
 *   single_counts  [E][R] int32, ACCUMULATED.
 * Integer sums: the result does not depend on their order.  Calls that
 * accumulate into the same tables must not run concurrently.
 * Errors: MOE_EINVAL, MOE_EUNSUPPORTED (as moe_send_counts()). */
int moe_shuffle_fit(const int32_t* prev_idx, const int32_t* cur_idx, const int32_t* next_idx,
                    int64_t tokens, int n_experts, int top_k, int n_ranks,
                    const int32_t* placement_next, int32_t* pair_counts, int32_t* single_counts,
                    void* stream);

/* Prediction: scores[t][r] = sum over the token's pairs (a, b), a's slot then
 * b's, of pair_counts[a][b][r] / n_ab when n_ab = sum_r pair_counts[a][b][r]
 * is at least min_obs (and positive), else of single_counts[b][r] / n_b (n_b
 * = sum_r single_counts[b][r]; nothing when n_b = 0).  fp64 in that order,
 * one rounding to fp32 per score.
 *   scores  [T][R] fp32 out.
 * Errors: MOE_EINVAL (min_obs < 0, null pointers), MOE_EUNSUPPORTED. */
int moe_shuffle_predict(const int32_t* prev_idx, const int32_t* cur_idx, int64_t tokens,
                        int n_experts, int top_k, int n_ranks, const int32_t* pair_counts,
                        const int32_t* single_counts, int min_obs, float* scores, void* stream);

/* Host.  Assignment: every rank owns exactly T/R tokens (T % R == 0).  Tokens
 * are taken in decreasing confidence = (largest score) / (sum of scores) (0
 * for an all-zero row; fp64 from the fp32 scores; ties to the lower token
 * index), each to its highest-scoring rank that still has room (ties to the
 * lower rank).  Synchronous; host memory only.
 *   scores  host [T][R] fp32;  owner  host [T] int32 out.
 * Errors: MOE_EINVAL (T % R != 0, null pointers), MOE_EUNSUPPORTED (R > 64, or its
 *         16 bytes per token of host tables could not be allocated). */
int moe_shuffle_assign(const float* scores, int64_t tokens, int n_ranks, int32_t* owner);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_H_ */
