/*
 * CPU oracle for the MoE layer forward pass and its backward.  TEST
 * INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  The HIP library never links, includes or calls it, and
 * this file includes nothing from the HIP library: the two share no code.
 *
 * It is written to be read against the pages it follows, not to be fast:
 * plain per-token loops, fp32 storage, fp64 accumulation, no blocking, no
 * fusion, no reordering beyond what each definition states.
 *
 * Pages cited (titles translated; original titles are given in the design
 * notes):
 *   [P1] "Optimising MoE with Triton: topk_gating operator fusion in practice"
 *   [P2] "SpMM in MoE: accelerating sparse experts with Triton kernels"
 *   [P4] "MoE architecture optimisation and SonicMoE practice"
 *   [P5] "Triton GPU kernel programming in practice"
 *
 * Pins (checked by the CPU tests, against things other than this file):
 *   softmax      - rows sum to 1; E=2 logistic closed form; equal row = 1/E
 *   top-K        - an independent full sort on tiny inputs, constructed ties
 *   weights      - sum to 1; K=1 gives 1; E=K=2 closed form; ratio property
 *   counts       - brute recount; sum = T*K; offsets = library cumulative sum
 *   permutation  - round trip, segment purity, ascending tokens in segments
 *   gather       - library fancy indexing
 *   expert FFN / combine / layer - E=1,K=1 equals a dense SwiGLU MLP built
 *                  from library matmuls; identical experts reduce to that MLP
 *                  for any routing; zero row; exact scaling by 2
 *   expert down  - reproduces expert FFN's y from its act; library matmul
 *   token rounding - hand-worked examples (tests/golden); the rounding rule's
 *                  nearest-multiple property; brute force that each expert
 *                  keeps its best-ranked candidates; M = 1 equals top-K;
 *                  weights sum to 1 with the logit ratios; the combine on
 *                  one-hot and token-index rows; identical experts give the
 *                  dense MLP built from library matmuls
 *   layer backward - central finite differences of oracle_layer for every
 *                  element of X, the logits and the three weight tensors; the
 *                  dS identity against the forward's act and a library matmul;
 *                  logit gradients sum to zero per token, zero for experts not
 *                  chosen, zero at K = 1 and for identical experts; exact
 *                  linearity in dout; exact bf16 widening
 * Every function here is pinned; none is "parity unpinned".
 *
 * Errors: every entry point returns 0 on success and a negative value on a
 * bad argument (null pointer, out-of-range size, non-finite logit).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* Widen one stored element to double.  bf16 is the upper half of an IEEE
 * binary32, so widening is exact: shift the 16 stored bits up by 16. */
static double load_elem(const void* base, int dtype, size_t i) {
    if (dtype == ORACLE_BF16) {
        uint32_t bits = ((uint32_t)((const uint16_t*)base)[i]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float*)base)[i];
}

/* [P1] §1 and [P5] §4: softmax over the E expert scores of one token, with the
 * maximum subtracted first for numerical stability ([P1] §4.1).  fp64. */
int oracle_softmax(const float* logits, int T, int E, double* probs) {
    if (!logits || !probs || T < 0 || E < 1) return -1;
    for (int t = 0; t < T; ++t) {
        const float* l = logits + (size_t)t * E;
        double m = -INFINITY;
        for (int e = 0; e < E; ++e) {
            if (!isfinite(l[e])) return -2;
            if ((double)l[e] > m) m = (double)l[e];
        }
        double s = 0.0;
        for (int e = 0; e < E; ++e) s += exp((double)l[e] - m);
        for (int e = 0; e < E; ++e) probs[(size_t)t * E + e] = exp((double)l[e] - m) / s;
    }
    return 0;
}

/* [P1] §1 (softmax then top-k over the expert axis), [P4] §1 (each token keeps
 * the K experts with the highest scores).  Selection is on the logits, which
 * orders experts exactly as their softmax probabilities do.  Slot 0 holds the
 * best expert; equal logits go to the lower expert index (float equality, so
 * -0.0 and +0.0 are equal).  Weights: the softmax probabilities of the chosen
 * experts, renormalised to sum to 1 over the K slots (fp64, rounded once).
 * Counts: [P4] §3.1, one count per (token, slot) added to its expert.
 * Offsets: exclusive prefix sum of the counts, with offsets[E] = T*K. */
int oracle_route(const float* logits, int T, int E, int K, int32_t* idx, float* w,
                 int32_t* counts, int32_t* offsets) {
    if (!logits || !idx || !w || !counts || !offsets) return -1;
    if (T < 0 || E < 1 || K < 1 || K > E) return -1;
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
    char* taken = (char*)malloc((size_t)E);
    if (!p || !taken) { free(p); free(taken); return -3; }
    int rc = 0;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int t = 0; t < T && rc == 0; ++t) {
        const float* l = logits + (size_t)t * E;
        rc = oracle_softmax(l, 1, E, p);
        if (rc) break;
        memset(taken, 0, (size_t)E);
        for (int k = 0; k < K; ++k) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e; /* strict: ties keep the lower e */
            }
            taken[best] = 1;
            idx[(size_t)t * K + k] = best;
        }
        double s = 0.0;
        for (int k = 0; k < K; ++k) s += p[idx[(size_t)t * K + k]];
        for (int k = 0; k < K; ++k) w[(size_t)t * K + k] = (float)(p[idx[(size_t)t * K + k]] / s);
        for (int k = 0; k < K; ++k) counts[idx[(size_t)t * K + k]] += 1;
    }
    free(p);
    free(taken);
    if (rc) return rc;
    int32_t run = 0;
    for (int e = 0; e < E; ++e) { offsets[e] = run; run += counts[e]; }
    offsets[E] = run;
    return 0;
}

/* [P2] §6 (each token row is duplicated once per selected expert) and [P4]
 * §2.2 (intermediates stored grouped by expert).  The expert-contiguous order
 * is a stable counting sort of the row-major (token, slot) list: walk experts
 * in ascending order, and inside an expert walk tokens in ascending order.
 * sorted_pair[p] = t*K + k, inv[t*K + k] = p. */
int oracle_permute(const int32_t* idx, int T, int E, int K, int32_t* sorted_pair, int32_t* inv) {
    if (!idx || !sorted_pair || !inv || T < 0 || E < 1 || K < 1) return -1;
    for (size_t q = 0; q < (size_t)T * K; ++q)
        if (idx[q] < 0 || idx[q] >= E) return -1;
    int32_t p = 0;
    for (int e = 0; e < E; ++e)
        for (int t = 0; t < T; ++t)
            for (int k = 0; k < K; ++k)
                if (idx[(size_t)t * K + k] == e) {
                    sorted_pair[p] = t * K + k;
                    inv[(size_t)t * K + k] = p;
                    ++p;
                }
    return 0;
}

/* Gather step of [P4] §1: row p of the expert-ordered input is the token row
 * that (token, slot) pair sorted_pair[p] came from.  A pure byte copy. */
int oracle_gather_rows(const void* X, int elem_bytes, int T, int d, int K,
                       const int32_t* sorted_pair, void* Xp) {
    if (!X || !sorted_pair || !Xp || elem_bytes < 1 || T < 0 || d < 0 || K < 1) return -1;
    size_t row = (size_t)d * elem_bytes;
    for (size_t p = 0; p < (size_t)T * K; ++p) {
        int32_t q = sorted_pair[p];
        if (q < 0 || q >= T * K) return -1;
        memcpy((char*)Xp + p * row, (const char*)X + (size_t)(q / K) * row, row);
    }
    return 0;
}

/* One expert's two-layer MLP with SwiGLU on one input row ([P4] §1: the first
 * layer's output passes through SiLU, H = SiLU(W1 X); [P4] §2.2: the SwiGLU
 * activation is applied to that product, gated by the W3 branch).
 *   h1[j] = sum_i x[i] W1[i,j],  h3[j] = sum_i x[i] W3[i,j]          (fp64)
 *   a[j]  = SiLU(h1[j]) * h3[j],  SiLU(z) = z / (1 + exp(-z))     (stored fp32)
 *   y[c]  = sum_j a[j] W2[j,c]                            (fp64, stored fp32)
 * W1, W3 are [d, n] and W2 is [n, d] for this expert, row-major. */
static void expert_row(const void* x, size_t xoff, int dtype, const void* W1, const void* W3,
                       const void* W2, size_t woff13, size_t woff2, int d, int n, double* h1,
                       double* h3, float* a, float* y) {
    for (int j = 0; j < n; ++j) { h1[j] = 0.0; h3[j] = 0.0; }
    for (int i = 0; i < d; ++i) {
        double xi = load_elem(x, dtype, xoff + (size_t)i);
        for (int j = 0; j < n; ++j) {
            h1[j] += xi * load_elem(W1, dtype, woff13 + (size_t)i * n + j);
            h3[j] += xi * load_elem(W3, dtype, woff13 + (size_t)i * n + j);
        }
    }
    for (int j = 0; j < n; ++j) a[j] = (float)(h1[j] / (1.0 + exp(-h1[j])) * h3[j]);
    double* acc = (double*)malloc(sizeof(double) * (size_t)d);
    for (int c = 0; c < d; ++c) acc[c] = 0.0;
    for (int j = 0; j < n; ++j) {
        double aj = (double)a[j];
        for (int c = 0; c < d; ++c) acc[c] += aj * load_elem(W2, dtype, woff2 + (size_t)j * d + c);
    }
    for (int c = 0; c < d; ++c) y[c] = (float)acc[c];
    free(acc);
}

/* Grouped expert MLP over expert-ordered rows ([P4] §1 GEMM step).  Row r of
 * Xp belongs to expert row_expert[r]; only the rows listed in `rows` (or all
 * `nrows` rows when rows == NULL) are computed.  act is [nsel, n], y is
 * [nsel, d], in the order of `rows`. */
int oracle_expert_ffn(const void* Xp, int dtype, int nrows, const int32_t* row_expert,
                      const int32_t* rows, int nsel, const void* W1, const void* W3,
                      const void* W2, int E, int d, int n, float* act, float* y) {
    if (!Xp || !row_expert || !W1 || !W3 || !W2 || !act || !y) return -1;
    if (nrows < 0 || nsel < 0 || E < 1 || d < 1 || n < 1) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int s = 0; s < nsel; ++s) {
        int r = rows ? rows[s] : s;
        if (r < 0 || r >= nrows || row_expert[r] < 0 || row_expert[r] >= E) { bad |= 1; continue; }
        int e = row_expert[r];
        double* h1 = (double*)malloc(sizeof(double) * (size_t)n);
        double* h3 = (double*)malloc(sizeof(double) * (size_t)n);
        expert_row(Xp, (size_t)r * d, dtype, W1, W3, W2, (size_t)e * d * n, (size_t)e * n * d, d, n,
                   h1, h3, act + (size_t)s * n, y + (size_t)s * d);
        free(h1);
        free(h3);
    }
    return bad ? -1 : 0;
}

/* The second layer alone ([P4] section 1: the expert MLP's second GEMM):
 * y[r, c] = sum_j act[r, j] W2[e_r][j, c] in fp64, stored fp32, where act is
 * given in the storage dtype (fp32, or bf16 widened exactly).  Equals the y
 * of oracle_expert_ffn when fed that function's act. */
int oracle_expert_down(const void* act, int dtype, int nrows, const int32_t* row_expert,
                       const void* W2, int E, int d, int n, float* y) {
    if (!act || !row_expert || !W2 || !y || nrows < 0 || E < 1 || d < 1 || n < 1) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
    for (int r = 0; r < nrows; ++r) {
        const int e = row_expert[r];
        if (e < 0 || e >= E) { bad |= 1; continue; }
        double* acc = (double*)calloc((size_t)d, sizeof(double));
        for (int j = 0; j < n; ++j) {
            const double aj = load_elem(act, dtype, (size_t)r * n + j);
            for (int c = 0; c < d; ++c) acc[c] += aj * load_elem(W2, dtype, (size_t)e * n * d + (size_t)j * d + c);
        }
        for (int c = 0; c < d; ++c) y[(size_t)r * d + c] = (float)acc[c];
        free(acc);
    }
    return bad ? -1 : 0;
}

/* Scatter / aggregation step ([P4] §1; [P2] §1 and §6: the outputs of the
 * selected experts are combined as a gate-weighted average).  With the
 * renormalised weights summing to 1 this is a weighted sum:
 *   out[t,c] = sum_k w[t,k] * Y[inv[t*K+k], c],  summed over k in order in fp64. */
int oracle_combine(const float* Y, const float* w, const int32_t* inv, int T, int d, int K,
                   float* out) {
    if (!Y || !w || !inv || !out || T < 0 || d < 0 || K < 1) return -1;
    for (int t = 0; t < T; ++t)
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += (double)w[(size_t)t * K + k] * (double)Y[(size_t)inv[(size_t)t * K + k] * d + c];
            out[(size_t)t * d + c] = (float)acc;
        }
    return 0;
}

/* The whole layer for a subset of tokens, as a per-token loop over the
 * selected experts: route the token, run each selected expert's MLP on the
 * token row, accumulate the gate-weighted outputs ([P4] §1 Router -> Experts
 * -> Aggregator).  It does not use the permutation at all.  tokens == NULL
 * means all T tokens; out is [ntok, d] in the order of `tokens`. */
int oracle_layer(const void* X, int dtype, const float* logits, const void* W1, const void* W3,
                 const void* W2, int T, int d, int E, int K, int n, const int32_t* tokens,
                 int ntok, float* out) {
    if (!X || !logits || !W1 || !W3 || !W2 || !out) return -1;
    if (T < 0 || d < 1 || E < 1 || K < 1 || K > E || n < 1 || ntok < 0) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int s = 0; s < ntok; ++s) {
        int t = tokens ? tokens[s] : s;
        if (t < 0 || t >= T) { bad |= 1; continue; }
        int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
        float* w = (float*)malloc(sizeof(float) * (size_t)K);
        int32_t* cnt = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
        int32_t* off = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
        double* h1 = (double*)malloc(sizeof(double) * (size_t)n);
        double* h3 = (double*)malloc(sizeof(double) * (size_t)n);
        float* a = (float*)malloc(sizeof(float) * (size_t)n);
        float* y = (float*)malloc(sizeof(float) * (size_t)d);
        double* acc = (double*)calloc((size_t)d, sizeof(double));
        if (oracle_route(logits + (size_t)t * E, 1, E, K, idx, w, cnt, off) != 0) bad |= 1;
        else
            for (int k = 0; k < K; ++k) {
                int e = idx[k];
                expert_row(X, (size_t)t * d, dtype, W1, W3, W2, (size_t)e * d * n,
                           (size_t)e * n * d, d, n, h1, h3, a, y);
                for (int c = 0; c < d; ++c) acc[c] += (double)w[k] * (double)y[c];
            }
        for (int c = 0; c < d; ++c) out[(size_t)s * d + c] = (float)acc[c];
        free(idx); free(w); free(cnt); free(off); free(h1); free(h3); free(a); free(y); free(acc);
    }
    return bad ? -1 : 0;
}

/* Router projection, the step upstream of the gate: page [P1] section 2.1
 * starts its fused flow from the logit computation, and page [P2] section 6
 * computes the gate logits with a linear layer over the token's features.
 * logits[t,e] = sum_i X[t,i] * Wr[i,e] (+ bias[e] when bias is not NULL),
 * summed in fp64 in index order, bias added last, rounded once to fp32.
 * X is [T,d] in dtype; Wr is [d,E] fp32; bias is [E] fp32. */
int oracle_router(const void* X, int dtype, const float* Wr, const float* bias, int T, int d, int E,
                  float* logits) {
    if (!X || !Wr || !logits || T < 0 || d < 1 || E < 1) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            double s = 0.0;
            for (int i = 0; i < d; ++i) s += load_elem(X, dtype, (size_t)t * d + i) * (double)Wr[(size_t)i * E + e];
            if (bias) s += (double)bias[e];
            logits[(size_t)t * E + e] = (float)s;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Token Rounding, the routing variant of [P4] section 3.  Section 3.1: the
 * per-expert token counts of ordinary top-K routing are rounded to a multiple
 * of the tile size M, up or down, and a second sort by score decides which
 * tokens an expert drops or takes on, so that every expert's row count is a
 * whole number of tiles.  Section 3.2: the rounding goes to the nearest
 * multiple (a remainder of exactly M/2 rounds up), the routing weights are
 * renormalised by a softmax over what each token keeps, and one expert may be
 * limited to a number of tiles (that section names 2M tokens).
 *
 * Readings taken where the pages leave a step open:
 *   - the counts rounded are those of oracle_route's top-K;
 *   - a target above T (an expert cannot take a token twice) rounds down;
 *   - cap_tiles > 0 limits a target to cap_tiles * M rows; 0 means no limit;
 *   - the second sort ranks tokens for expert e by logit[t,e] descending,
 *     then token index ascending.  An expert whose target is below its count
 *     keeps its best routed tokens; one whose target is above keeps all of
 *     them and takes on the best tokens not routed to it;
 *   - a token left with no expert contributes a zero output row;
 *   - rows are laid out expert by expert, tokens ascending inside an expert.
 * ------------------------------------------------------------------------- */
typedef struct {
    float l;
    int32_t t;
} tr_cand;

/* Better candidate first: larger logit, then lower token index. */
static int tr_cand_cmp(const void* a, const void* b) {
    const tr_cand* x = (const tr_cand*)a;
    const tr_cand* y = (const tr_cand*)b;
    if (x->l > y->l) return -1;
    if (x->l < y->l) return 1;
    return (x->t > y->t) - (x->t < y->t);
}

/* Rows an expert with f routed tokens ends up with. */
int32_t oracle_tr_target(int32_t f, int M, int T, int cap_tiles) {
    int64_t r = (((int64_t)f + M / 2) / M) * M;
    if (r > T) r -= M;
    if (cap_tiles > 0 && r > (int64_t)cap_tiles * M) r = (int64_t)cap_tiles * M;
    return (int32_t)r;
}

/* Outputs: counts_r[E], offsets_r[E+1] (exclusive sums, offsets_r[E] = rows),
 * row_tok[rows] (token of each row), slot_row[T,E] (row of (t,e) or -1) and
 * slot_w[T,E] (weight of (t,e), 0 where not kept):
 *   w[t,e] = exp(l[t,e] - m) / sum_{e' kept by t} exp(l[t,e'] - m),
 * m the largest kept logit of t, in fp64, rounded once.  rows_cap is the room
 * in row_tok; more rows than that is an error (-4). */
int oracle_token_round(const float* logits, int T, int E, int K, int M, int cap_tiles,
                       int32_t* counts_r, int32_t* offsets_r, int32_t* row_tok, int64_t rows_cap,
                       int32_t* slot_row, float* slot_w) {
    if (!logits || !counts_r || !offsets_r || !row_tok || !slot_row || !slot_w) return -1;
    if (T < 0 || E < 1 || K < 1 || K > E || M < 1 || cap_tiles < 0 || rows_cap < 0) return -1;
    const size_t TE = (size_t)T * E;
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * ((size_t)T * K + 1));
    float* w = (float*)malloc(sizeof(float) * ((size_t)T * K + 1));
    int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
    char* routed = (char*)calloc(TE + 1, 1);
    char* kept = (char*)calloc(TE + 1, 1);
    tr_cand* cand = (tr_cand*)malloc(sizeof(tr_cand) * ((size_t)T + 1));
    int rc = (idx && w && counts && offsets && routed && kept && cand) ? 0 : -3;
    if (rc == 0) rc = oracle_route(logits, T, E, K, idx, w, counts, offsets);
    if (rc == 0) {
        for (size_t q = 0; q < (size_t)T * K; ++q) routed[(q / K) * E + idx[q]] = 1;
        int64_t run = 0;
        for (int e = 0; e < E; ++e) {
            const int32_t f = counts[e];
            const int32_t r = oracle_tr_target(f, M, T, cap_tiles);
            int n = 0;
            if (r <= f) {
                /* keep the r best routed tokens */
                for (int t = 0; t < T; ++t)
                    if (routed[(size_t)t * E + e]) { cand[n].l = logits[(size_t)t * E + e]; cand[n].t = t; ++n; }
                qsort(cand, (size_t)n, sizeof(tr_cand), tr_cand_cmp);
                for (int j = 0; j < r; ++j) kept[(size_t)cand[j].t * E + e] = 1;
            } else {
                /* keep every routed token and take on the r - f best others */
                for (int t = 0; t < T; ++t) {
                    if (routed[(size_t)t * E + e]) kept[(size_t)t * E + e] = 1;
                    else { cand[n].l = logits[(size_t)t * E + e]; cand[n].t = t; ++n; }
                }
                qsort(cand, (size_t)n, sizeof(tr_cand), tr_cand_cmp);
                for (int j = 0; j < r - f; ++j) kept[(size_t)cand[j].t * E + e] = 1;
            }
            counts_r[e] = r;
            offsets_r[e] = (int32_t)run;
            run += r;
        }
        offsets_r[E] = (int32_t)run;
        if (run > rows_cap) rc = -4;
    }
    if (rc == 0) {
        int32_t p = 0;
        for (int e = 0; e < E; ++e)
            for (int t = 0; t < T; ++t) {
                if (kept[(size_t)t * E + e]) { row_tok[p] = t; slot_row[(size_t)t * E + e] = p; ++p; }
                else slot_row[(size_t)t * E + e] = -1;
            }
        for (int t = 0; t < T; ++t) {
            const float* l = logits + (size_t)t * E;
            double m = -INFINITY;
            for (int e = 0; e < E; ++e)
                if (kept[(size_t)t * E + e] && (double)l[e] > m) m = (double)l[e];
            double s = 0.0;
            for (int e = 0; e < E; ++e)
                if (kept[(size_t)t * E + e]) s += exp((double)l[e] - m);
            for (int e = 0; e < E; ++e)
                slot_w[(size_t)t * E + e] = kept[(size_t)t * E + e] ? (float)(exp((double)l[e] - m) / s) : 0.0f;
        }
    }
    free(idx); free(w); free(counts); free(offsets); free(routed); free(kept); free(cand);
    return rc;
}

/* Combine after Token Rounding: the aggregation of [P4] section 1 over the
 * experts a token kept, in ascending expert order, in fp64:
 *   out[t,c] = sum_{e: slot_row[t,e] >= 0} slot_w[t,e] * Y[slot_row[t,e], c]. */
int oracle_tr_combine(const float* Y, const int32_t* slot_row, const float* slot_w, int T, int E, int d,
                      int64_t nrows, float* out) {
    if (!Y || !slot_row || !slot_w || !out || T < 0 || E < 1 || d < 0 || nrows < 0) return -1;
    for (int t = 0; t < T; ++t)
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int e = 0; e < E; ++e) {
                const int32_t r = slot_row[(size_t)t * E + e];
                if (r < 0) continue;
                if (r >= nrows) return -1;
                acc += (double)slot_w[(size_t)t * E + e] * (double)Y[(size_t)r * d + c];
            }
            out[(size_t)t * d + c] = (float)acc;
        }
    return 0;
}

/* The layer after Token Rounding, per token: each expert the token kept runs
 * its MLP on the token row and the outputs are summed with the kept weights,
 * in ascending expert order ([P4] section 1, Router -> Experts -> Aggregator,
 * with the routing of section 3).  Only slot_row's sign is used: the rows
 * themselves play no part.  tokens == NULL means all T tokens. */
int oracle_tr_layer(const void* X, int dtype, const int32_t* slot_row, const float* slot_w, const void* W1,
                    const void* W3, const void* W2, int T, int d, int E, int n, const int32_t* tokens, int ntok,
                    float* out) {
    if (!X || !slot_row || !slot_w || !W1 || !W3 || !W2 || !out) return -1;
    if (T < 0 || d < 1 || E < 1 || n < 1 || ntok < 0) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int s = 0; s < ntok; ++s) {
        const int t = tokens ? tokens[s] : s;
        if (t < 0 || t >= T) { bad |= 1; continue; }
        double* h1 = (double*)malloc(sizeof(double) * (size_t)n);
        double* h3 = (double*)malloc(sizeof(double) * (size_t)n);
        float* a = (float*)malloc(sizeof(float) * (size_t)n);
        float* y = (float*)malloc(sizeof(float) * (size_t)d);
        double* acc = (double*)calloc((size_t)d, sizeof(double));
        for (int e = 0; e < E; ++e) {
            if (slot_row[(size_t)t * E + e] < 0) continue;
            expert_row(X, (size_t)t * d, dtype, W1, W3, W2, (size_t)e * d * n, (size_t)e * n * d, d, n, h1, h3,
                       a, y);
            const double we = (double)slot_w[(size_t)t * E + e];
            for (int c = 0; c < d; ++c) acc[c] += we * (double)y[c];
        }
        for (int c = 0; c < d; ++c) out[(size_t)s * d + c] = (float)acc[c];
        free(h1); free(h3); free(a); free(y); free(acc);
    }
    return bad ? -1 : 0;
}

/* ---------------------------------------------------------------------------
 * Backward of the layer: the gradient of oracle_layer's output with respect
 * to X, the router logits and the expert weights, given dout = dL/d(out).
 * [P4] section 2.2 names the two products the backward needs beside the
 * weight gradients, dH (through the SwiGLU) and dS, the gradient of the
 * routing scores; [P4] section 5 measures the backward pass.  Per token t and
 * slot k with expert e, weight w_k, and g = dout[t]:
 *   h1 = x W1[e], h3 = x W3[e], s1 = SiLU(h1), a = s1 * h3, y = a W2[e]
 *   dw[t,k]  = <g, y>                      (dS; equals <g W2[e]^T, a>, the
 *                                            form [P4] section 2.2 uses)
 *   da       = w_k (g W2[e]^T)
 *   dW2[e]  += w_k a^T g
 *   dh3      = da * s1,   dh1 = da * h3 * SiLU'(h1),
 *              SiLU'(z) = sig(z) (1 + z (1 - sig(z))),  sig(z) = 1 / (1 + e^-z)
 *   dX[t]   += dh1 W1[e]^T + dh3 W3[e]^T
 *   dW1[e]  += x^T dh1,   dW3[e] += x^T dh3
 * The weights are the softmax of the K chosen logits renormalised over them,
 * so for a chosen expert j
 *   dlogits[t, idx_j] = w_j (dw_j - sum_k w_k dw_k)
 * and 0 for the others (the top-K choice itself is piecewise constant).
 * The routing is oracle_route's.  Everything is summed in fp64 in index order
 * (tokens ascending for the weight gradients) and rounded once to fp32; the
 * activations are not rounded to fp32 in between, so this is the gradient of
 * the real-valued function that oracle_layer evaluates.  Sized for small
 * inputs: it holds fp64 copies of the three weight gradients.
 * dw may be NULL. */
/* One token of the backward: its routing, dX row (gx, d doubles), its K
 * routing-weight gradients (dwk) and, when gW1 is not NULL, its contribution
 * to the three weight gradients (fp64 accumulators).  Scratch: h1, h3, a, ga,
 * dh1, dh3 of n doubles.  Returns oracle_route's status. */
static int bwd_token(const void* X, int dtype, const float* logits, const void* W1, const void* W3, const void* W2,
                     int t, int d, int E, int K, int n, const float* g, int32_t* idx, float* w, int32_t* cnt,
                     int32_t* off, double* h1, double* h3, double* a, double* ga, double* dh1, double* dh3,
                     double* gx, double* dwk, double* gW1, double* gW3, double* gW2) {
    const int rc = oracle_route(logits + (size_t)t * E, 1, E, K, idx, w, cnt, off);
    if (rc) return rc;
    const size_t xoff = (size_t)t * d;
    for (int i = 0; i < d; ++i) gx[i] = 0.0;
    for (int k = 0; k < K; ++k) {
        const int e = idx[k];
        const size_t o13 = (size_t)e * d * n, o2 = (size_t)e * n * d;
        const double wk = (double)w[k];
        for (int j = 0; j < n; ++j) { h1[j] = 0.0; h3[j] = 0.0; }
        for (int i = 0; i < d; ++i) {
            const double xi = load_elem(X, dtype, xoff + i);
            for (int j = 0; j < n; ++j) {
                h1[j] += xi * load_elem(W1, dtype, o13 + (size_t)i * n + j);
                h3[j] += xi * load_elem(W3, dtype, o13 + (size_t)i * n + j);
            }
        }
        double dws = 0.0;
        for (int j = 0; j < n; ++j) {
            a[j] = h1[j] / (1.0 + exp(-h1[j])) * h3[j];
            double sacc = 0.0;
            for (int c = 0; c < d; ++c) sacc += (double)g[c] * load_elem(W2, dtype, o2 + (size_t)j * d + c);
            ga[j] = sacc;  /* (g W2[e]^T)[j] */
        }
        /* dS = <g, y> with y = a W2[e], summed over the output columns */
        for (int c = 0; c < d; ++c) {
            double yc = 0.0;
            for (int j = 0; j < n; ++j) yc += a[j] * load_elem(W2, dtype, o2 + (size_t)j * d + c);
            dws += (double)g[c] * yc;
        }
        dwk[k] = dws;
        if (gW2)
            for (int j = 0; j < n; ++j)
                for (int c = 0; c < d; ++c) gW2[o2 + (size_t)j * d + c] += wk * a[j] * (double)g[c];
        for (int j = 0; j < n; ++j) {
            const double sig = 1.0 / (1.0 + exp(-h1[j]));
            const double s1 = h1[j] * sig;
            const double da = wk * ga[j];
            dh3[j] = da * s1;
            dh1[j] = da * h3[j] * sig * (1.0 + h1[j] * (1.0 - sig));
        }
        for (int i = 0; i < d; ++i) {
            const double xi = load_elem(X, dtype, xoff + i);
            double sacc = 0.0;
            for (int j = 0; j < n; ++j) {
                sacc += dh1[j] * load_elem(W1, dtype, o13 + (size_t)i * n + j) +
                        dh3[j] * load_elem(W3, dtype, o13 + (size_t)i * n + j);
                if (gW1) {
                    gW1[o13 + (size_t)i * n + j] += xi * dh1[j];
                    gW3[o13 + (size_t)i * n + j] += xi * dh3[j];
                }
            }
            gx[i] += sacc;
        }
    }
    return 0;
}

/* The logit gradient of one token from its weights and weight gradients. */
static void bwd_logits(const int32_t* idx, const float* w, const double* dwk, int E, int K, float* dl) {
    double mean = 0.0;
    for (int k = 0; k < K; ++k) mean += (double)w[k] * dwk[k];
    for (int e = 0; e < E; ++e) dl[e] = 0.0f;
    for (int k = 0; k < K; ++k) dl[idx[k]] = (float)((double)w[k] * (dwk[k] - mean));
}

int oracle_layer_backward(const void* X, int dtype, const float* logits, const void* W1, const void* W3,
                          const void* W2, int T, int d, int E, int K, int n, const float* dout, float* dX,
                          float* dlogits, float* dW1, float* dW3, float* dW2, float* dw) {
    if (!X || !logits || !W1 || !W3 || !W2 || !dout || !dX || !dlogits || !dW1 || !dW3 || !dW2) return -1;
    if (T < 0 || d < 1 || E < 1 || K < 1 || K > E || n < 1) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    const size_t wn = (size_t)E * d * n;
    double* gW1 = (double*)calloc(wn, sizeof(double));
    double* gW3 = (double*)calloc(wn, sizeof(double));
    double* gW2 = (double*)calloc(wn, sizeof(double));
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    float* w = (float*)malloc(sizeof(float) * (size_t)K);
    int32_t* cnt = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    int32_t* off = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
    double* scr = (double*)malloc(sizeof(double) * (size_t)(6 * n + d + K));
    int rc = 0;
    if (!gW1 || !gW3 || !gW2 || !idx || !w || !cnt || !off || !scr) rc = -3;
    for (int t = 0; t < T && rc == 0; ++t) {
        double* gx = scr + 6 * (size_t)n;
        double* dwk = gx + d;
        rc = bwd_token(X, dtype, logits, W1, W3, W2, t, d, E, K, n, dout + (size_t)t * d, idx, w, cnt, off, scr,
                       scr + n, scr + 2 * (size_t)n, scr + 3 * (size_t)n, scr + 4 * (size_t)n, scr + 5 * (size_t)n,
                       gx, dwk, gW1, gW3, gW2);
        if (rc) break;
        for (int i = 0; i < d; ++i) dX[(size_t)t * d + i] = (float)gx[i];
        bwd_logits(idx, w, dwk, E, K, dlogits + (size_t)t * E);
        if (dw)
            for (int k = 0; k < K; ++k) dw[(size_t)t * K + k] = (float)dwk[k];
    }
    if (rc == 0)
        for (size_t q = 0; q < wn; ++q) {
            dW1[q] = (float)gW1[q];
            dW3[q] = (float)gW3[q];
            dW2[q] = (float)gW2[q];
        }
    free(gW1); free(gW3); free(gW2); free(idx); free(w); free(cnt); free(off); free(scr);
    return rc;
}

/* The same backward for a subset of tokens, without the weight gradients:
 * rows s of dX [ntok, d], dlogits [ntok, E] and dw [ntok, K] belong to token
 * tokens[s]; dout is the full [T, d].  For sampled checks of large layers. */
int oracle_layer_backward_rows(const void* X, int dtype, const float* logits, const void* W1, const void* W3,
                               const void* W2, int T, int d, int E, int K, int n, const float* dout,
                               const int32_t* tokens, int ntok, float* dX, float* dlogits, float* dw) {
    if (!X || !logits || !W1 || !W3 || !W2 || !dout || !tokens || !dX || !dlogits || !dw) return -1;
    if (T < 0 || d < 1 || E < 1 || K < 1 || K > E || n < 1 || ntok < 0) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int s = 0; s < ntok; ++s) {
        const int t = tokens[s];
        if (t < 0 || t >= T) { bad |= 1; continue; }
        int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
        float* w = (float*)malloc(sizeof(float) * (size_t)K);
        int32_t* cnt = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
        int32_t* off = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
        double* scr = (double*)malloc(sizeof(double) * (size_t)(6 * n + d + K));
        double* gx = scr + 6 * (size_t)n;
        double* dwk = gx + d;
        if (bwd_token(X, dtype, logits, W1, W3, W2, t, d, E, K, n, dout + (size_t)t * d, idx, w, cnt, off, scr,
                      scr + n, scr + 2 * (size_t)n, scr + 3 * (size_t)n, scr + 4 * (size_t)n, scr + 5 * (size_t)n,
                      gx, dwk, NULL, NULL, NULL) != 0)
            bad |= 1;
        else {
            for (int i = 0; i < d; ++i) dX[(size_t)s * d + i] = (float)gx[i];
            bwd_logits(idx, w, dwk, E, K, dlogits + (size_t)s * E);
            for (int k = 0; k < K; ++k) dw[(size_t)s * K + k] = (float)dwk[k];
        }
        free(idx); free(w); free(cnt); free(off); free(scr);
    }
    return bad ? -1 : 0;
}

/* Slices of the expert-weight gradients, for checks of large layers whose full
 * gradients the fp64 accumulators of oracle_layer_backward could not hold.
 * For pair p = (e, j) = (experts[p], cols[p]) it writes column j of dW1[e] and
 * of dW3[e] (d values each: dW1[e][i][j] for i = 0..d-1) and row j of dW2[e]
 * (d values: dW2[e][j][c]), into rows p of dW1c, dW3c and dW2r [npair, d].
 * Same definition and summation order as oracle_layer_backward ([P4] section
 * 2.2): over the assignments (t, k) with idx[t,k] == e, tokens ascending,
 *   h1 = x W1[e][:,j], h3 = x W3[e][:,j], sig = 1/(1+e^-h1), s1 = h1 sig,
 *   a = s1 h3, da = w_k (g W2[e][j,:]^T),
 *   dh1 = da h3 sig (1 + h1 (1 - sig)), dh3 = da s1,
 *   dW1[e][:,j] += x dh1,  dW3[e][:,j] += x dh3,  dW2[e][j,:] += w_k a g,
 * in fp64, rounded once to fp32.  The routing is oracle_route's over all T. */
int oracle_weight_grad_slices(const void* X, int dtype, const float* logits, const void* W1, const void* W3,
                              const void* W2, int T, int d, int E, int K, int n, const float* dout,
                              const int32_t* experts, const int32_t* cols, int npair, float* dW1c, float* dW3c,
                              float* dW2r) {
    if (!X || !logits || !W1 || !W3 || !W2 || !dout || !experts || !cols || !dW1c || !dW3c || !dW2r) return -1;
    if (T < 0 || d < 1 || E < 1 || K < 1 || K > E || n < 1 || npair < 0) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    for (int p = 0; p < npair; ++p)
        if (experts[p] < 0 || experts[p] >= E || cols[p] < 0 || cols[p] >= n) return -1;
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * ((size_t)T * K + 1));
    float* w = (float*)malloc(sizeof(float) * ((size_t)T * K + 1));
    int32_t* cnt = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    int32_t* off = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int rc = (!idx || !w || !cnt || !off) ? -3 : oracle_route(logits, T, E, K, idx, w, cnt, off);
    int bad = 0;
    if (rc == 0) {
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
        for (int p = 0; p < npair; ++p) {
            const int e = experts[p], j = cols[p];
            const size_t o13 = (size_t)e * d * n, o2 = (size_t)e * n * d;
            double* acc = (double*)calloc(3 * (size_t)d, sizeof(double));
            if (!acc) { bad |= 1; continue; }
            double* g1 = acc;
            double* g3 = acc + d;
            double* g2 = acc + 2 * (size_t)d;
            for (int t = 0; t < T; ++t)
                for (int k = 0; k < K; ++k) {
                    if (idx[(size_t)t * K + k] != e) continue;
                    const size_t xoff = (size_t)t * d;
                    const float* g = dout + (size_t)t * d;
                    const double wk = (double)w[(size_t)t * K + k];
                    double h1 = 0.0, h3 = 0.0, ga = 0.0;
                    for (int i = 0; i < d; ++i) {
                        const double xi = load_elem(X, dtype, xoff + i);
                        h1 += xi * load_elem(W1, dtype, o13 + (size_t)i * n + j);
                        h3 += xi * load_elem(W3, dtype, o13 + (size_t)i * n + j);
                    }
                    for (int c = 0; c < d; ++c) ga += (double)g[c] * load_elem(W2, dtype, o2 + (size_t)j * d + c);
                    const double sig = 1.0 / (1.0 + exp(-h1));
                    const double s1 = h1 * sig;
                    const double a = h1 / (1.0 + exp(-h1)) * h3;
                    const double da = wk * ga;
                    const double dh3 = da * s1;
                    const double dh1 = da * h3 * sig * (1.0 + h1 * (1.0 - sig));
                    for (int i = 0; i < d; ++i) {
                        const double xi = load_elem(X, dtype, xoff + i);
                        g1[i] += xi * dh1;
                        g3[i] += xi * dh3;
                    }
                    for (int c = 0; c < d; ++c) g2[c] += wk * a * (double)g[c];
                }
            for (int i = 0; i < d; ++i) {
                dW1c[(size_t)p * d + i] = (float)g1[i];
                dW3c[(size_t)p * d + i] = (float)g3[i];
                dW2r[(size_t)p * d + i] = (float)g2[i];
            }
            free(acc);
        }
    }
    free(idx); free(w); free(cnt); free(off);
    if (rc) return rc;
    return bad ? -3 : 0;
}

