/*
 * CPU oracle for per-GPU MoE expert-parallel dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no source with the HIP kernels.
 *
 * Plain, slow, single-threaded loops in the order the definitions are stated.
 * Floating point that the pages leave open is done in fp64 and rounded once,
 * except the combine, which is a fixed chain of fp32 fused multiply-adds (see
 * oracle_combine_rows).
 *
 * Sources (page title, then section):
 *  [EC]  "Expert Coupling in MoE Pretraining: Reducing All-to-All Overhead with
 *        Correlated Placement and Token Shuffling" (summary page).
 *        - "Background": each token goes to its top-k experts.
 *        - "Method 1: Correlated Expert Placement + Deduplicating Dispatcher":
 *          plain dispatch repeats a token's row for each of its experts; the
 *          deduplicating variant writes it once per rank the token needs, with
 *          the ids and gates of the token's experts on that rank attached;
 *          W[e][e'] is the number of tokens choosing both e and e'; a GPU
 *          holds E/EP experts.
 *  [DD]  "DODOCO: MoE AlltoAll Traffic Matrices on Real Text" (dataset card).
 *        - "Setup": contiguous placement, rank r holds experts r*E/R..;
 *          the counts are the dispatcher's per-destination input splits.
 *        - "Reading the counts": one count per token-expert assignment, even when
 *          several experts share a destination; each row sums to tokens*top-k;
 *          each rank's expert-block sum is its receive total.
 *        - "send_matrices.csv columns": combine returns the same volumes in
 *          reverse.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *  - gates: softmax over the k selected logits, in fp64, rounded once to fp32;
 *  - top-k order: logit descending, ties to the lower expert index, IEEE
 *    comparison (so -0.0 ties +0.0);
 *  - send buffer order: rank ascending, then expert id, then token (non-dedup);
 *    rank ascending, then token (dedup);
 *  - dedup row weight: sum of that rank's gates in ascending expert order, fp64,
 *    rounded once to fp32;
 *  - combine: sum over the distinct rows serving a token, in ascending row
 *    index, of weight*row as a chain of fp32 fused multiply-adds starting from
 *    -0.0, rounded once to bf16 (round to nearest even);
 *  - W's diagonal counts the tokens selecting e.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- route --- */

typedef struct {
    float logit;
    int32_t expert;
} oracle_cand;

/* Order: larger logit first; equal logits (IEEE ==, so -0.0 == +0.0): lower
 * expert index first. */
static int oracle_cand_cmp(const void* pa, const void* pb) {
    const oracle_cand* a = (const oracle_cand*)pa;
    const oracle_cand* b = (const oracle_cand*)pb;
    if (a->logit > b->logit) return -1;
    if (a->logit < b->logit) return 1;
    return (a->expert > b->expert) - (a->expert < b->expert);
}

/* [EC] "Background": each token is routed to its top-k experts.
 * idx[t][j] = the j-th expert of token t in (logit desc, index asc) order.
 * gate[t][j] = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0), fp64, rounded once. */
int oracle_route_topk(const float* logits, int64_t tokens, int n_experts, int top_k,
                      int32_t* idx, float* gate) {
    if (top_k < 1 || top_k > n_experts) return 1;
    oracle_cand* c = (oracle_cand*)malloc(sizeof(oracle_cand) * (size_t)n_experts);
    double* ex = (double*)malloc(sizeof(double) * (size_t)top_k);
    if (!c || !ex) { free(c); free(ex); return 2; }
    for (int64_t t = 0; t < tokens; ++t) {
        const float* row = logits + t * n_experts;
        for (int e = 0; e < n_experts; ++e) {
            c[e].logit = row[e];
            c[e].expert = e;
        }
        qsort(c, (size_t)n_experts, sizeof(oracle_cand), oracle_cand_cmp);
        const double l0 = (double)c[0].logit;
        double s = 0.0;
        for (int j = 0; j < top_k; ++j) {
            ex[j] = exp((double)c[j].logit - l0);
            s += ex[j];
        }
        for (int j = 0; j < top_k; ++j) {
            idx[t * top_k + j] = c[j].expert;
            gate[t * top_k + j] = (float)(ex[j] / s);
        }
    }
    free(c);
    free(ex);
    return 0;
}

/* The same selection; gate[t][j] = exp(l_j - l_0) / sum over all E experts e
 * of exp(l_e - l_0): the softmax over every logit, taken at the selected
 * experts and not renormalised (the other reading of "routing
 * probabilities").  fp64, summed in expert order, rounded once. */
int oracle_route_topk_softmax_all(const float* logits, int64_t tokens, int n_experts, int top_k,
                                  int32_t* idx, float* gate) {
    int rc = oracle_route_topk(logits, tokens, n_experts, top_k, idx, gate);
    if (rc) return rc;
    for (int64_t t = 0; t < tokens; ++t) {
        const float* row = logits + t * n_experts;
        const double l0 = (double)row[idx[t * top_k]];
        double s = 0.0;
        for (int e = 0; e < n_experts; ++e) s += exp((double)row[e] - l0);
        for (int j = 0; j < top_k; ++j)
            gate[t * top_k + j] = (float)(exp((double)row[idx[t * top_k + j]] - l0) / s);
    }
    return 0;
}

/* ------------------------------------------------------- counts, offsets --- */

/* [DD] "Reading the counts" and [EC] "Method 1".
 * expert_counts[e] = #(t, j) with idx[t][j] == e.
 * Non-dedup: rank_counts[r] = sum of expert_counts over the experts placed on r.
 * Dedup:     rank_counts[r] = #tokens with at least one selected expert on r.
 * rank_offsets = exclusive scan of rank_counts (R+1 entries).
 * expert_offsets[e] = rank_offsets[place[e]] + counts of the experts on the same
 * rank with a lower id (the start of e's segment in the non-dedup buffer). */
int oracle_send_counts(const int32_t* idx, int64_t tokens, int n_experts, int top_k,
                       int n_ranks, const int32_t* place, int dedup,
                       int32_t* expert_counts, int32_t* rank_counts,
                       int32_t* rank_offsets, int32_t* expert_offsets) {
    for (int e = 0; e < n_experts; ++e) expert_counts[e] = 0;
    for (int r = 0; r < n_ranks; ++r) rank_counts[r] = 0;
    for (int64_t t = 0; t < tokens; ++t)
        for (int j = 0; j < top_k; ++j) expert_counts[idx[t * top_k + j]] += 1;
    if (!dedup) {
        for (int e = 0; e < n_experts; ++e) rank_counts[place[e]] += expert_counts[e];
    } else {
        for (int64_t t = 0; t < tokens; ++t) {
            for (int r = 0; r < n_ranks; ++r) {
                int hit = 0;
                for (int j = 0; j < top_k; ++j)
                    if (place[idx[t * top_k + j]] == r) hit = 1;
                rank_counts[r] += hit;
            }
        }
    }
    rank_offsets[0] = 0;
    for (int r = 0; r < n_ranks; ++r) rank_offsets[r + 1] = rank_offsets[r] + rank_counts[r];
    if (expert_offsets) {
        for (int e = 0; e < n_experts; ++e) {
            int32_t off = rank_offsets[place[e]];
            for (int e2 = 0; e2 < e; ++e2)
                if (place[e2] == place[e]) off += expert_counts[e2];
            expert_offsets[e] = off;
        }
    }
    return 0;
}

/* --------------------------------------------------- non-dedup dispatch --- */

/* [EC] "Method 1" (conventional top-k dispatch) and [DD] "Reading the counts":
 * one row per (token, expert).  Rows are written in the order the send buffer
 * is laid out: rank ascending, expert ascending within a rank, token ascending
 * within an expert.  Walking tokens in order and bumping a per-expert cursor
 * that starts at expert_offsets[e] produces exactly that order. */
int oracle_dispatch(const uint8_t* x, const int32_t* idx, const float* gate,
                    int64_t tokens, int row_bytes, int n_experts, int top_k,
                    const int32_t* expert_offsets, uint8_t* send, int32_t* row_token,
                    int32_t* row_expert, float* row_weight, int32_t* slot_row) {
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_experts);
    if (!cursor) return 2;
    for (int e = 0; e < n_experts; ++e) cursor[e] = expert_offsets[e];
    for (int64_t t = 0; t < tokens; ++t) {
        for (int j = 0; j < top_k; ++j) {
            const int e = idx[t * top_k + j];
            const int32_t p = cursor[e]++;
            if (send) memcpy(send + (int64_t)p * row_bytes, x + t * row_bytes, (size_t)row_bytes);
            row_token[p] = (int32_t)t;
            row_expert[p] = e;
            row_weight[p] = gate[t * top_k + j];
            slot_row[t * top_k + j] = p;
        }
    }
    free(cursor);
    return 0;
}

/* ------------------------------------------------------- dedup dispatch --- */

/* [EC] "Method 1", deduplicating dispatcher: one row per distinct (token,
 * destination rank).  The row carries the ids of that rank's selected experts
 * (ascending, padded with -1), their gates (aligned, padded with 0) and
 * row_weight = the sum of those gates.  Send buffer order: rank ascending,
 * token ascending within a rank.  slot_row[t][j] = the row serving slot j. */
int oracle_dispatch_dedup(const uint8_t* x, const int32_t* idx, const float* gate,
                          int64_t tokens, int row_bytes, int n_experts, int top_k,
                          int n_ranks, const int32_t* place, const int32_t* rank_offsets,
                          uint8_t* send, int32_t* row_token, int32_t* row_experts,
                          float* row_gates, float* row_weight, int32_t* slot_row,
                          int32_t* n_rows) {
    (void)n_experts;
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_ranks);
    int* sel = (int*)malloc(sizeof(int) * (size_t)top_k);
    if (!cursor || !sel) { free(cursor); free(sel); return 2; }
    for (int r = 0; r < n_ranks; ++r) cursor[r] = rank_offsets[r];
    for (int64_t t = 0; t < tokens; ++t) {
        const int32_t* ti = idx + t * top_k;
        for (int r = 0; r < n_ranks; ++r) {
            /* the slots of token t whose expert lives on rank r */
            int ns = 0;
            for (int j = 0; j < top_k; ++j)
                if (place[ti[j]] == r) sel[ns++] = j;
            if (ns == 0) continue;
            /* order those slots by expert id (insertion sort, ns <= k) */
            for (int a = 1; a < ns; ++a) {
                int v = sel[a], b = a - 1;
                while (b >= 0 && ti[sel[b]] > ti[v]) { sel[b + 1] = sel[b]; --b; }
                sel[b + 1] = v;
            }
            const int32_t p = cursor[r]++;
            if (send) memcpy(send + (int64_t)p * row_bytes, x + t * row_bytes, (size_t)row_bytes);
            row_token[p] = (int32_t)t;
            double wsum = 0.0;
            for (int c = 0; c < top_k; ++c) {
                if (c < ns) {
                    row_experts[(int64_t)p * top_k + c] = ti[sel[c]];
                    row_gates[(int64_t)p * top_k + c] = gate[t * top_k + sel[c]];
                    wsum += (double)gate[t * top_k + sel[c]];
                } else {
                    row_experts[(int64_t)p * top_k + c] = -1;
                    row_gates[(int64_t)p * top_k + c] = 0.0f;
                }
            }
            row_weight[p] = (float)wsum;
            for (int c = 0; c < ns; ++c) slot_row[t * top_k + sel[c]] = p;
        }
    }
    *n_rows = rank_offsets[n_ranks];
    free(cursor);
    free(sel);
    return 0;
}

/* ---------------------------------------------- receive-side expansion --- */

/* [EC] "Method 1": a deduplicated row carries the ids and routing
 * probabilities of every selected expert on its destination rank, so the
 * receiving rank hands the row to each of those experts.  Expansion lays the
 * received rows out per expert: for every row p < n_rows and every listed
 * expert e (ids >= 0; -1 is padding), one copy of row p.  Order: rank
 * ascending, expert id ascending within a rank, row ascending within an
 * expert (the order of the conventional dispatcher's buffer).
 * expert_counts[e] = number of rows listing e; rank_counts[r] = the sum over the
 * experts on r; rank_offsets = its exclusive scan; expert_offsets[e] = start of
 * e's segment.  Per expanded row q: exp_row[q] = source row, exp_expert[q] =
 * expert, exp_gate[q] = that expert's gate on the row.  row_slot[p][c] = the
 * expanded row of (p, listed column c); -1 for padding and for every row
 * p >= n_rows up to `capacity`. */
int oracle_expand_dedup(const uint8_t* rows, const int32_t* row_experts,
                        const float* row_gates, int64_t n_rows, int64_t capacity,
                        int row_bytes, int n_experts, int top_k, int n_ranks,
                        const int32_t* place, int32_t* expert_counts, int32_t* rank_counts,
                        int32_t* rank_offsets, int32_t* expert_offsets, uint8_t* expanded,
                        int32_t* exp_row, int32_t* exp_expert, float* exp_gate,
                        int32_t* row_slot) {
    for (int e = 0; e < n_experts; ++e) expert_counts[e] = 0;
    for (int r = 0; r < n_ranks; ++r) rank_counts[r] = 0;
    for (int64_t p = 0; p < n_rows; ++p)
        for (int c = 0; c < top_k; ++c) {
            const int32_t e = row_experts[p * top_k + c];
            if (e >= 0) expert_counts[e] += 1;
        }
    for (int e = 0; e < n_experts; ++e) rank_counts[place[e]] += expert_counts[e];
    rank_offsets[0] = 0;
    for (int r = 0; r < n_ranks; ++r) rank_offsets[r + 1] = rank_offsets[r] + rank_counts[r];
    for (int e = 0; e < n_experts; ++e) {
        int32_t off = rank_offsets[place[e]];
        for (int e2 = 0; e2 < e; ++e2)
            if (place[e2] == place[e]) off += expert_counts[e2];
        expert_offsets[e] = off;
    }
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_experts);
    if (!cursor) return 2;
    for (int e = 0; e < n_experts; ++e) cursor[e] = expert_offsets[e];
    for (int64_t i = 0; i < capacity * top_k; ++i) row_slot[i] = -1;
    for (int64_t p = 0; p < n_rows; ++p) {
        for (int c = 0; c < top_k; ++c) {
            const int32_t e = row_experts[p * top_k + c];
            if (e < 0) continue;
            const int32_t q = cursor[e]++;
            if (expanded)
                memcpy(expanded + (int64_t)q * row_bytes, rows + p * row_bytes, (size_t)row_bytes);
            exp_row[q] = (int32_t)p;
            exp_expert[q] = e;
            exp_gate[q] = row_gates[p * top_k + c];
            row_slot[p * top_k + c] = q;
        }
    }
    free(cursor);
    return 0;
}

/* -------------------------------------------------------------- combine --- */

/* bf16 value nearest to d, ties to even (IEEE round to nearest even), as bits.
 * Written from the definition: the quantum of a bf16 with leading-bit exponent
 * p is 2^(p-7) (7 fraction bits), with p clamped at -126 below (subnormals);
 * d / quantum is exact, nearbyint rounds it half-to-even in the default mode. */
uint16_t oracle_bf16_from_double(double d) {
    if (isnan(d)) return (uint16_t)(signbit(d) ? 0xFFC0u : 0x7FC0u);
    if (isinf(d)) return (uint16_t)(signbit(d) ? 0xFF80u : 0x7F80u);
    if (d == 0.0) return (uint16_t)(signbit(d) ? 0x8000u : 0x0000u);
    int ex;
    (void)frexp(d, &ex);          /* |d| = m * 2^ex, 0.5 <= m < 1 */
    int lead = ex - 1;            /* exponent of d's leading bit */
    if (lead < -126) lead = -126;
    const double q = ldexp(1.0, lead - 7);
    const double r = nearbyint(d / q) * q;
    const double max_bf16 = ldexp(255.0, 127 - 7);   /* 0x7F7F = (2 - 2^-7) * 2^127 */
    if (fabs(r) > max_bf16) return (uint16_t)(signbit(d) ? 0xFF80u : 0x7F80u);
    if (r == 0.0) return (uint16_t)(signbit(d) ? 0x8000u : 0x0000u);
    const float f = (float)r;     /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* The fp32 value of a bf16 bit pattern: bf16 is the top half of an fp32. */
static float oracle_bf16_to_float(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* bf16 nearest to the fp32 value f, ties to even.  Every fp32 value is exact
 * in fp64, so this is the rounding above; a NaN keeps its sign and the top of
 * its payload and is made quiet. */
uint16_t oracle_bf16_from_float(float f) {
    if (isnan(f)) {
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        return (uint16_t)((u >> 16) | 0x0040u);
    }
    return oracle_bf16_from_double((double)f);
}

/* fp8 E4M3 in the OCP 8-bit floating point format: sign, 4 exponent bits
 * (bias 7), 3 mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6;
 * no infinities; S.1111.111 is NaN.  Decoded exactly into a double. */
double oracle_e4m3_to_double(uint8_t b) {
    const int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* [EC] "The Communication Bottleneck" (dispatch, experts, combine) and [DD]
 * "send_matrices.csv columns" (combine is the reverse exchange): each token's
 * output is the weighted sum of the rows that served it.
 * out[t][h] = bf16( sum over the distinct rows r in slot_row[t][.] (r >= 0)
 *                   of w[r] * rows[r][h] ).
 * The pages fix no order or precision for this sum; the reading taken: rows
 * in ascending index, acc = -0.0f, then acc = fmaf(w[r], rows[r][h], acc) for
 * each row (fp32, one rounding per step), and one round-to-nearest-even of acc
 * to bf16.  -0.0 as the start keeps an all-(-0) sum at -0 and makes the empty
 * sum -0.  w == NULL means weight 1 for every row.  Rows of fp8 E4M3 are
 * decoded exactly (every E4M3 value is an fp32 value). */
static int oracle_combine_rows(const void* rows, int fp8, const float* w, const int32_t* slot_row,
                               int64_t tokens, int hidden_dim, int top_k, uint16_t* out) {
    int32_t* rs = (int32_t*)malloc(sizeof(int32_t) * (size_t)top_k);
    if (!rs) return 2;
    for (int64_t t = 0; t < tokens; ++t) {
        /* distinct non-negative rows, ascending */
        int nr = 0;
        for (int j = 0; j < top_k; ++j) {
            const int32_t r = slot_row[t * top_k + j];
            if (r < 0) continue;
            int seen = 0;
            for (int i = 0; i < nr; ++i) if (rs[i] == r) seen = 1;
            if (!seen) rs[nr++] = r;
        }
        for (int a = 1; a < nr; ++a) {
            int32_t v = rs[a];
            int b = a - 1;
            while (b >= 0 && rs[b] > v) { rs[b + 1] = rs[b]; --b; }
            rs[b + 1] = v;
        }
        for (int h = 0; h < hidden_dim; ++h) {
            float acc = -0.0f;
            for (int i = 0; i < nr; ++i) {
                const float wr = w ? w[rs[i]] : 1.0f;
                const int64_t at = (int64_t)rs[i] * hidden_dim + h;
                const float y = fp8 ? (float)oracle_e4m3_to_double(((const uint8_t*)rows)[at])
                                    : oracle_bf16_to_float(((const uint16_t*)rows)[at]);
                acc = fmaf(wr, y, acc);
            }
            out[t * hidden_dim + h] = oracle_bf16_from_float(acc);
        }
    }
    free(rs);
    return 0;
}

int oracle_combine(const uint16_t* rows, const float* w, const int32_t* slot_row,
                   int64_t tokens, int hidden_dim, int top_k, uint16_t* out) {
    return oracle_combine_rows(rows, 0, w, slot_row, tokens, hidden_dim, top_k, out);
}

/* The same sum over rows of fp8 E4M3 values (the dispatch precision may be
 * one byte per element: [DD] "Reading the counts"); output bf16. */
int oracle_combine_fp8(const uint8_t* rows, const float* w, const int32_t* slot_row,
                       int64_t tokens, int hidden_dim, int top_k, uint16_t* out) {
    return oracle_combine_rows(rows, 1, w, slot_row, tokens, hidden_dim, top_k, out);
}

/* --------------------------------------------------------- co-selection --- */

/* [EC] "Method 1": W[e][e'] counts the tokens that select both e and e'
 * (e != e'); the diagonal W[e][e] counts the tokens selecting e.  Only the first
 * `tokens` tokens are used ("Correlation Formation and Stability": ~4096 tokens
 * suffice).  Accumulates into W. */
int oracle_coselect(const int32_t* idx, int64_t tokens, int n_experts, int top_k,
                    int32_t* W) {
    for (int64_t t = 0; t < tokens; ++t) {
        const int32_t* ti = idx + t * top_k;
        for (int a = 0; a < top_k; ++a) {
            for (int b = 0; b < top_k; ++b) {
                /* a == b: the diagonal; a != b: each ordered pair once */
                W[(int64_t)ti[a] * n_experts + ti[b]] += 1;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------- placement search --- */

/* [EC] "Method 1", correlated placement: starting from a placement (contiguous
 * unless given), swap experts between ranks to raise the co-location objective
 *   O(place) = sum over ordered pairs x != y with place[x] == place[y] of W[x][y]
 * while every rank keeps its E/R experts.  The page names a Kernighan-Lin-style
 * local search without printing it; this is the plainest reading: repeatedly
 * apply the swap (e, f), place[e] != place[f], e < f, with the largest gain,
 * ties to the lowest e then the lowest f, until no swap gains or max_swaps
 * swaps were made.
 * Gain of swapping e (rank a) and f (rank b), with
 *   A(x, r) = sum over y on r, y != x, of W[x][y] + W[y][x]:
 *   A(e, b) + A(f, a) - A(e, a) - A(f, b) - 2 (W[e][f] + W[f][e]).
 * Every A is summed afresh with plain loops for every candidate. */
static int64_t oracle_attach(const int32_t* W, int n, const int32_t* place, int x, int r) {
    int64_t s = 0;
    for (int y = 0; y < n; ++y)
        if (y != x && place[y] == r) s += (int64_t)W[(int64_t)x * n + y] + W[(int64_t)y * n + x];
    return s;
}

int64_t oracle_placement_objective(const int32_t* W, int n_experts, const int32_t* place) {
    int64_t o = 0;
    for (int x = 0; x < n_experts; ++x)
        for (int y = 0; y < n_experts; ++y)
            if (x != y && place[x] == place[y]) o += W[(int64_t)x * n_experts + y];
    return o;
}

int oracle_placement_search(const int32_t* W, int n_experts, int n_ranks, const int32_t* initial,
                            int max_swaps, int32_t* place, int64_t* objective, int* swaps) {
    const int n = n_experts;
    for (int e = 0; e < n; ++e) place[e] = initial ? initial[e] : e / (n / n_ranks);
    int done = 0;
    while (done < max_swaps) {
        int64_t best = 0;
        int be = -1, bf = -1;
        for (int e = 0; e < n; ++e) {
            for (int f = e + 1; f < n; ++f) {
                const int a = place[e], b = place[f];
                if (a == b) continue;
                const int64_t g = oracle_attach(W, n, place, e, b) + oracle_attach(W, n, place, f, a)
                                - oracle_attach(W, n, place, e, a) - oracle_attach(W, n, place, f, b)
                                - 2 * ((int64_t)W[(int64_t)e * n + f] + W[(int64_t)f * n + e]);
                if (g > best) { best = g; be = e; bf = f; }
            }
        }
        if (be < 0) break;
        const int t = place[be];
        place[be] = place[bf];
        place[bf] = t;
        ++done;
    }
    if (objective) *objective = oracle_placement_objective(W, n, place);
    if (swaps) *swaps = done;
    return 0;
}

/* ------------------------------------------------ token shuffle planner --- */

/* [EC] "Method 2: Token Shuffling", prediction.  The serving rank at layer
 * l+1 is guessed from the token's experts at layers l-1 and l, or from its
 * layer-l expert alone when that pair is rare.  Reading (no formula is
 * printed): on a
 * calibration batch, for every token, every expert c it selects at l+1 (rank
 * r = place_next[c]) and every pair (a, b) of its experts at l-1 and l,
 *   pair[a][b][r] += 1;   and for every b at l:  single[b][r] += 1.
 * Both tables accumulate (caller-zeroed int32). */
int oracle_shuffle_fit(const int32_t* prev, const int32_t* cur, const int32_t* next,
                       int64_t tokens, int n_experts, int top_k, int n_ranks,
                       const int32_t* place_next, int32_t* pair, int32_t* single) {
    const int E = n_experts, k = top_k, R = n_ranks;
    for (int64_t t = 0; t < tokens; ++t) {
        for (int jc = 0; jc < k; ++jc) {
            const int r = place_next[next[t * k + jc]];
            for (int ja = 0; ja < k; ++ja)
                for (int jb = 0; jb < k; ++jb) {
                    const int a = prev[t * k + ja], b = cur[t * k + jb];
                    pair[((int64_t)a * E + b) * R + r] += 1;
                }
            for (int jb = 0; jb < k; ++jb) single[(int64_t)cur[t * k + jb] * R + r] += 1;
        }
    }
    return 0;
}

/* Scores of every rank for every token: the sum over the token's (a, b) pairs,
 * in slot order (a's slot, then b's), of the pair's rank distribution
 * pair[a][b][r] / sum_r pair[a][b][r] when that sum is at least min_obs, else
 * of b's distribution single[b][r] / sum_r single[b][r] (nothing when b was
 * never seen).  fp64, one rounding to fp32 per score. */
int oracle_shuffle_predict(const int32_t* prev, const int32_t* cur, int64_t tokens,
                           int n_experts, int top_k, int n_ranks, const int32_t* pair,
                           const int32_t* single, int min_obs, float* scores) {
    const int E = n_experts, k = top_k, R = n_ranks;
    double* sc = (double*)malloc(sizeof(double) * (size_t)R);
    if (!sc) return 2;
    for (int64_t t = 0; t < tokens; ++t) {
        for (int r = 0; r < R; ++r) sc[r] = 0.0;
        for (int ja = 0; ja < k; ++ja) {
            for (int jb = 0; jb < k; ++jb) {
                const int a = prev[t * k + ja], b = cur[t * k + jb];
                const int32_t* pr = pair + ((int64_t)a * E + b) * R;
                int64_t n = 0;
                for (int r = 0; r < R; ++r) n += pr[r];
                if (n >= min_obs && n > 0) {
                    for (int r = 0; r < R; ++r) sc[r] += (double)pr[r] / (double)n;
                } else {
                    const int32_t* sr = single + (int64_t)b * R;
                    int64_t m = 0;
                    for (int r = 0; r < R; ++r) m += sr[r];
                    if (m > 0)
                        for (int r = 0; r < R; ++r) sc[r] += (double)sr[r] / (double)m;
                }
            }
        }
        for (int r = 0; r < R; ++r) scores[t * R + r] = (float)sc[r];
    }
    free(sc);
    return 0;
}

/* "Capacity Constraint": every rank owns exactly T/R tokens (T % R == 0);
 * tokens are taken in decreasing confidence = (largest score) / (sum of
 * scores) (0 for an all-zero row; computed in fp64 from the fp32 scores; ties
 * to the lower token index) and each goes to its highest-scoring rank that
 * still has room (ties to the lower rank). */
typedef struct { double conf; int64_t t; } oracle_conf;

static int oracle_conf_cmp(const void* pa, const void* pb) {
    const oracle_conf* a = (const oracle_conf*)pa;
    const oracle_conf* b = (const oracle_conf*)pb;
    if (a->conf > b->conf) return -1;
    if (a->conf < b->conf) return 1;
    return (a->t > b->t) - (a->t < b->t);
}

int oracle_shuffle_assign(const float* scores, int64_t tokens, int n_ranks, int32_t* owner) {
    const int R = n_ranks;
    if (tokens % R != 0) return 1;
    oracle_conf* c = (oracle_conf*)malloc(sizeof(oracle_conf) * (size_t)(tokens > 0 ? tokens : 1));
    int64_t* room = (int64_t*)malloc(sizeof(int64_t) * (size_t)R);
    if (!c || !room) { free(c); free(room); return 2; }
    for (int64_t t = 0; t < tokens; ++t) {
        double mx = 0.0, sum = 0.0;
        for (int r = 0; r < R; ++r) {
            const double v = (double)scores[t * R + r];
            sum += v;
            if (v > mx) mx = v;
        }
        c[t].conf = sum > 0.0 ? mx / sum : 0.0;
        c[t].t = t;
    }
    qsort(c, (size_t)tokens, sizeof(oracle_conf), oracle_conf_cmp);
    for (int r = 0; r < R; ++r) room[r] = tokens / R;
    for (int64_t i = 0; i < tokens; ++i) {
        const int64_t t = c[i].t;
        int best = -1;
        for (int r = 0; r < R; ++r) {
            if (room[r] == 0) continue;
            if (best < 0 || scores[t * R + r] > scores[t * R + best]) best = r;
        }
        owner[t] = best;
        room[best] -= 1;
    }
    free(c);
    free(room);
    return 0;
}
