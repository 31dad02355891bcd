/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE layer forward library, libmoe.so.
 *
 * The layer follows the problem statement of [P4] section 1: tokens
 * X in R^{T x d}, E expert scores per token, the K best experts kept per
 * token, and each expert a two-layer MLP whose first layer goes through SiLU
 * (SwiGLU: W1 and W3 are [d, n], W2 is [n, d]).  The forward pass is
 * gate -> histogram/offsets -> permute (gather) -> grouped expert MLP ->
 * combine (scatter), as in [P4] section 1 and [P2] section 6.
 *
 * Pages cited (titles translated):
 *   [P1] "Optimising MoE with Triton: topk_gating operator fusion in practice"
 *   [P2] "SpMM in MoE: accelerating sparse experts with Triton kernels"
 *   [P3] "Triton optimisation speeds up matrix computation for Mixture-of-Experts models"
 *   [P4] "MoE architecture optimisation and SonicMoE practice"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers unless stated; the caller owns every buffer.
 *    The library never allocates or frees memory and keeps no state between
 *    calls except a per-device cache of the compute-unit count.
 *  - Tensors are dense and row-major.  Expert weights are stacked expert-major:
 *    W1[e] starts at element e*d*n.  No biases.
 *  - `dtype` (moe_dtype) is the storage type of X, W1, W3, W2, Xp, Act, Y and
 *    out.  Router logits and gate weights are always fp32; indices int32.
 *    Arithmetic: fp32 accumulation; bf16 results are rounded to nearest-even.
 *  - Every device pointer must be 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work on it: no host<->device synchronisation, no copies.
 *  - Errors: a call returns a moe_status.  Arguments are validated before any
 *    launch; on a validation error nothing is launched and no output is
 *    touched.  MOE_ERR_HIP reports a failed launch.  Faults inside a kernel
 *    surface at the caller's next synchronisation.  moe_last_error() gives a
 *    human-readable reason for the last failure on the calling thread.
 *  - Router logits must be finite; non-finite logits give unspecified routing.
 *  - Supported sizes: 1 <= E <= 256, 1 <= K <= min(E, 8), T >= 1,
 *    T*K < 2^31; for the layer calls d and n are multiples of 128 (bf16) or
 *    of 64 (fp32), and T*K*max(d,n) < 2^40.  Outside these: MOE_ERR_UNSUPPORTED
 *    (or MOE_ERR_INVALID_ARG for values that are meaningless, such as K > E).
 *  - Calls that write the same buffers race if they overlap on different
 *    streams; calls on one stream are ordered.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,  /* null pointer, misalignment, meaningless size */
    MOE_ERR_UNSUPPORTED = 2,  /* valid but outside the supported sizes above */
    MOE_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
    MOE_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Static string naming a status code ("ok", "invalid argument", ...). */
const char* moe_status_string(int status);

/* Reason for the most recent non-OK status returned on this thread. */
const char* moe_last_error(void);

/* Workspace sizes in bytes (device memory, 256-byte aligned start) for the
 * calls that need one.  Return 0 for invalid sizes.
 * moe_workspace_bytes: one workspace that serves every forward-path call on
 * these sizes -- moe_route, moe_permute, moe_grouped_ffn (with its split),
 * moe_ffn_up, moe_ffn_down and moe_forward (the largest of their needs). */
size_t moe_workspace_bytes(int T, int d, int E, int K, int n, int dtype);
size_t moe_route_workspace_bytes(int T, int E, int K);
size_t moe_permute_workspace_bytes(int T, int E, int K);
size_t moe_forward_workspace_bytes(int T, int d, int E, int K, int n, int dtype);
/* Optional workspace of moe_grouped_ffn / moe_ffn_up / moe_ffn_down on the
 * current device (0 when the sizes take no split, e.g. fp32). */
size_t moe_ffn_workspace_bytes(int d, int n, int dtype);
/* Workspace of moe_router (0 when none is needed: fp32 X, or d % 256 != 0). */
size_t moe_router_workspace_bytes(int d, int E, int dtype);

/* Router projection, upstream of step 1: the router logits from the tokens.
 *   [P1] section 2.1: the fused gating flow starts from the logit
 *   computation; [P2] section 6: the gate logits are a linear layer over the
 *   token's features.
 * Semantics: logits[t,e] = sum_i X[t,i] * Wr[i,e] + bias[e] (no bias term when
 *   bias is NULL).
 * In:  X [T,d] in dtype (row-major), Wr [d,E] fp32 (row-major: expert index
 *      fastest), bias [E] fp32 or NULL.
 * Out: logits [T,E] fp32, the input of moe_route / moe_forward.
 * Precision: bf16 X with d % 256 == 0 runs on bf16 MFMA with each weight
 *   split into two bf16 terms (hi = bf16(w), lo = bf16(w - hi), so that
 *   |w - hi - lo| <= 2^-18 |w|) and fp32 accumulation; otherwise fp32 fused
 *   multiply-adds in index order.  The error is that of an fp32 dot product
 *   (over 2d terms on the MFMA path), plus at most 2^-18 * S from the split,
 *   S = sum_i |X[t,i] Wr[i,e]|; the tests hold it to 2^-16 * S.
 * Workspace: moe_router_workspace_bytes(d,E,dtype) bytes (the split weights,
 *   rewritten on every call); NULL allowed when that is 0.  X and ws must be
 *   16-byte aligned on the MFMA path.
 * Sizes: T >= 1, d >= 1, 1 <= E <= 256, T*E < 2^31.  Deterministic.
 */
int moe_router(const void* X, int dtype, int T, int d, int E, const float* Wr, const float* bias,
               float* logits, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_route -- steps 1 and 2: fused softmax top-K gate, per-expert histogram
 * and exclusive prefix offsets.
 *   [P1] section 1: softmax over the expert axis, then top-k, then a per-expert
 *   accumulation, fused into one pass ([P1] section 2.1); [P4] section 1: the
 *   K best of E scores per token; [P4] section 3.1: per-expert token counts.
 * Semantics (per token t):
 *   topk_idx[t,0..K-1]: the K experts with the largest logits, best first;
 *     equal logits go to the lower expert index (-0.0 equals +0.0).
 *   topk_w[t,k] = softmax(logits[t])[idx] renormalised over the K slots,
 *     i.e. exp(l_k - l_0) / sum_j exp(l_j - l_0).
 *   counts[e] = number of (t,k) with topk_idx[t,k] == e.
 *   offsets[e] = sum_{e' < e} counts[e'], offsets[E] = T*K  (E+1 entries).
 * In:  logits [T,E] fp32.
 * Out: topk_idx [T,K] int32, topk_w [T,K] fp32, counts [E] int32,
 *      offsets [E+1] int32.
 * Workspace: moe_route_workspace_bytes(T,E,K) bytes (per-chunk counts).
 * Deterministic: integer histogram, no floating-point atomics.
 */
int moe_route(const float* logits, int T, int E, int K, int32_t* topk_idx, float* topk_w,
              int32_t* counts, int32_t* offsets, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_route_noalloc -- moe_route for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same semantics, arguments (less the workspace), kernels
 * and results as moe_route.
 * Scratch: the per-chunk expert counts live in a static device array of
 *   MOE_ROUTE_NOALLOC_SCRATCH_BYTES (1 MiB) that each GPU the library runs on
 *   holds until the process ends; its address is looked up on the first call
 *   on a device.  No call allocates or frees memory.  A chunk is 256 tokens
 *   (1024 when T > 65536), and ceil(T / chunk) * E * 4 bytes must fit the
 *   scratch (e.g. T = 262144 with E = 256, or T = 2^20 with E = 256), else
 *   MOE_ERR_UNSUPPORTED and nothing is launched.
 * Concurrency: every call on a GPU shares that GPU's scratch, so calls that
 *   overlap on one GPU (on different streams, or from different threads on
 *   different streams) race.  Calls ordered on one stream are safe.
 */
#define MOE_ROUTE_NOALLOC_SCRATCH_BYTES (1u << 20)
int moe_route_noalloc(const float* logits, int T, int E, int K, int32_t* topk_idx, float* topk_w, int32_t* counts,
                      int32_t* offsets, void* stream);

/*
 * moe_permute -- step 3: token rows into expert-contiguous order.
 *   [P2] section 6: each token row is repeated once per selected expert;
 *   [P4] section 1 (gather) and section 2.2 (intermediates grouped by expert).
 * Order: a stable counting sort of the row-major (t,k) list by expert: rows of
 * expert e occupy [offsets[e], offsets[e+1]) in ascending token order, where
 * offsets is the exclusive scan of the expert histogram of topk_idx (exactly
 * what moe_route returns).  The placement is derived from topk_idx itself, so
 * no offsets argument is taken and no stale offsets can misplace a row.
 * In:  X [T,d] (dtype; d*sizeof(dtype) a multiple of 16 bytes),
 *      topk_idx [T,K] int32 with entries in [0,E) and the K entries of a
 *      token distinct (as moe_route produces).  Entries outside [0,E) are
 *      skipped: their rows are not placed and their inv entries not written.
 * Out: sorted_pair [T*K] int32 (= t*K + k at each expert-ordered position p),
 *      inv [T*K] int32 (inv[t*K+k] = p), Xp [T*K, d] (dtype), Xp[p] = X[t].
 * Workspace: moe_permute_workspace_bytes(T,E,K) bytes.
 */
int moe_permute(const void* X, int dtype, int T, int d, int E, int K, const int32_t* topk_idx,
                int32_t* sorted_pair, int32_t* inv, void* Xp, void* ws, size_t ws_bytes,
                void* stream);

/*
 * moe_grouped_ffn -- step 4: grouped GEMM over all experts in one launch per
 * layer ([P3] technical innovations: many independent GEMMs in one kernel;
 * persistent design: as many workgroups as the GPU holds, pulling tiles),
 * with the SwiGLU activation fused into the first GEMM's epilogue ([P4]
 * section 2.2).
 *   For expert e, rows r in [offsets[e], offsets[e] + counts[e]) of Xp:
 *     Act[r] = SiLU(Xp[r] W1[e]) * (Xp[r] W3[e]),  SiLU(z) = z / (1 + e^-z)
 *     Y[r]   = Act[r] W2[e]
 *   fp32 accumulation; Act and Y stored in dtype.
 * In:  Xp [T*K,d], W1 [E,d,n], W3 [E,d,n], W2 [E,n,d], counts [E],
 *      offsets [E+1].
 * Out: Act [T*K,n], Y [T*K,d].  The ragged tile schedule is derived from
 *      counts on the device.
 * Workspace (optional): NULL, or moe_ffn_workspace_bytes(d,n,dtype) bytes.
 *      With it, the tiles of each GEMM's last, partial round are split along K
 *      over the otherwise idle workgroups; the fp32 parts are added in a fixed
 *      order, so results stay deterministic (they may differ from the unsplit
 *      ones by fp32 rounding).  It also holds the counters from which the
 *      workgroups of each XCD claim their tiles one at a time (cleared by the
 *      library before each GEMM), so that workgroups that drew short tiles
 *      take more; which workgroup computes a tile does not change the result.
 *      Calls that share one workspace must not overlap.  A non-NULL ws that
 *      is too small is MOE_ERR_WORKSPACE.
 */
int moe_grouped_ffn(const void* Xp, const void* W1, const void* W3, const void* W2, int dtype,
                    int T, int d, int E, int K, int n, const int32_t* counts,
                    const int32_t* offsets, void* Act, void* Y, void* ws, size_t ws_bytes,
                    void* stream);

/*
 * moe_ffn_up -- step 4a alone: the SwiGLU GEMM of moe_grouped_ffn.
 *   Act[r] = SiLU(Xp[r] W1[e]) * (Xp[r] W3[e]) for rows r of expert e
 *   ([P4] section 1 first layer through SiLU; section 2.2 SwiGLU epilogue).
 * Arguments and layouts as for moe_grouped_ffn.  Out: Act [T*K,n].
 */
int moe_ffn_up(const void* Xp, const void* W1, const void* W3, int dtype, int T, int d, int E, int K,
               int n, const int32_t* counts, const int32_t* offsets, void* Act, void* ws,
               size_t ws_bytes, void* stream);

/*
 * moe_ffn_down -- step 4b alone: the down-projection GEMM of moe_grouped_ffn.
 *   Y[r] = Act[r] W2[e] for rows r of expert e ([P4] section 1 second layer).
 * In: Act [T*K,n] (dtype), W2 [E,n,d], counts [E], offsets [E+1].
 * Out: Y [T*K,d].  Workspace as for moe_grouped_ffn.
 */
int moe_ffn_down(const void* Act, const void* W2, int dtype, int T, int d, int E, int K, int n,
                 const int32_t* counts, const int32_t* offsets, void* Y, void* ws, size_t ws_bytes,
                 void* stream);

/*
 * moe_combine -- step 5: gate-weighted combine back to token order ([P4]
 * section 1 scatter; [P2] sections 1 and 6: the selected experts' outputs are
 * averaged with the gate weights).  A gather-sum by token, no atomics:
 *   out[t] = sum_{k=0}^{K-1} topk_w[t,k] * Y[inv[t*K+k]]
 * summed in k order in fp32 and rounded once to dtype.
 * In:  Y [T*K,d] (dtype), topk_w [T,K] fp32, inv [T*K] int32.
 * Out: out [T,d] (dtype).
 */
int moe_combine(const void* Y, const float* topk_w, const int32_t* inv, int dtype, int T, int d,
                int K, void* out, void* stream);

/*
 * moe_forward -- the whole layer: moe_route, moe_permute, moe_grouped_ffn and
 * moe_combine on one stream, with the permutation's per-chunk counts reused
 * from the gate.  Results equal those of the four calls made in sequence.
 * In:  X [T,d], logits [T,E], W1, W3 [E,d,n], W2 [E,n,d].
 * Out: out [T,d].
 * Optional outputs (may be NULL, then they live in the workspace):
 *      topk_idx [T,K], topk_w [T,K], counts [E], offsets [E+1],
 *      sorted_pair [T*K], inv [T*K].
 * Workspace: moe_forward_workspace_bytes(T,d,E,K,n,dtype) bytes; it also holds
 *      Act [T*K,n] and Y [T*K,d], and Xp [T*K,d] only where the SwiGLU GEMM
 *      cannot read the X rows in place (bf16 with d % 256 == 0, n % 128 == 0,
 *      d*n*2 < 2^31 and T*d*2 < 2^31 gather them; other sizes and fp32 take
 *      the copy).
 */
int moe_forward(const void* X, const float* logits, const void* W1, const void* W3,
                const void* W2, int dtype, int T, int d, int E, int K, int n, void* out,
                int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                int32_t* sorted_pair, int32_t* inv, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_route_x -- the router projection and steps 1-2 from the tokens: logits
 * = X Wr (+ bias) as moe_router computes them, then the gate, histogram and
 * offsets of moe_route on those logits.
 *   [P1] section 2.1: one fused pass from the logit computation through the
 *   softmax to the top-k; [P2] section 6: the gate logits are a linear layer;
 *   [P4] section 1: the K best of E scores per token.
 * Fused where bf16 X, d % 256 == 0 and E <= 64: one kernel computes the
 *   logits of a 32-token tile on MFMA and runs the gate on them from LDS, so
 *   the logits never travel through memory (unless `logits` asks for them).
 *   Elsewhere the router and the gate run one after the other, through the
 *   caller's `logits` or workspace room.
 * In:  X [T,d] (dtype), Wr [d,E] fp32, bias [E] fp32 or NULL.
 * Out: topk_idx [T,K], topk_w [T,K], counts [E], offsets [E+1] as moe_route;
 *      logits [T,E] fp32 (optional, NULL = not written) equal, bit for bit,
 *      to what moe_router writes for the same arguments, and the routing is
 *      that of moe_route on them (weights within 1e-5 relative).
 * Workspace: moe_route_x_workspace_bytes(T,d,E,K,dtype) bytes (the split
 *      weights and the expert counts, rewritten on every call).
 * Sizes: those of moe_route and moe_router.
 */
size_t moe_route_x_workspace_bytes(int T, int d, int E, int K, int dtype);
int moe_route_x(const void* X, int dtype, int T, int d, int E, int K, const float* Wr, const float* bias,
                float* logits, int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets, void* ws,
                size_t ws_bytes, void* stream);

/*
 * moe_forward_x -- the whole layer from the tokens and the router weights:
 * moe_route_x in place of moe_route, then moe_forward's steps 3-5.
 *   [P1] section 2.1 (the fused gate starts from the logit computation) and
 *   [P4] section 1 (the layer).
 * In:  X [T,d], Wr [d,E] fp32, bias [E] fp32 or NULL, W1, W3 [E,d,n],
 *      W2 [E,n,d].
 * Out: out [T,d]; the results of moe_forward given the logits moe_router
 *      writes for X, Wr and bias.
 * Optional outputs (may be NULL): logits [T,E] as moe_route_x, and those of
 *      moe_forward.
 * Workspace: moe_forward_x_workspace_bytes(T,d,E,K,n,dtype) bytes.
 * Sizes and errors: those of moe_forward and moe_router.
 */
size_t moe_forward_x_workspace_bytes(int T, int d, int E, int K, int n, int dtype);
int moe_forward_x(const void* X, const float* Wr, const float* bias, const void* W1, const void* W3, const void* W2,
                  int dtype, int T, int d, int E, int K, int n, void* out, float* logits, int32_t* topk_idx,
                  float* topk_w, int32_t* counts, int32_t* offsets, int32_t* sorted_pair, int32_t* inv, void* ws,
                  size_t ws_bytes, void* stream);

/*
 * Token Rounding -- the routing variant of [P4] section 3.  Section 3.1: the
 * per-expert counts of top-K routing are rounded to whole tiles of M rows and
 * a second sort by score picks which tokens each expert drops or takes on.
 * Section 3.2: rounding to the nearest multiple (a remainder of exactly M/2
 * rounds up), a per-expert limit (cap_tiles tiles; 0 = none; the page names
 * 2M tokens) and the weights renormalised by a softmax over what each token
 * keeps.  Readings where the pages leave a step open:
 *   - f_e = rows of expert e under top-K (the `counts` of moe_route);
 *     r_e = M*floor((f_e + floor(M/2)) / M), less M if that exceeds T, then
 *     at most cap_tiles*M when cap_tiles > 0;
 *   - tokens are ranked for expert e by logits[t,e] descending, then t
 *     ascending; if r_e <= f_e the expert keeps its r_e best routed tokens,
 *     else all its routed tokens plus the r_e - f_e best others;
 *   - w[t,e] = exp(l[t,e] - m) / sum over the experts t kept of exp(l - m),
 *     m the largest kept logit (fp32); a token that kept none gets a zero row.
 * Plan layout: rows expert by expert (offsets_r), tokens ascending inside an
 * expert; row_tok[row] = token; slot_row[t,e] = the row of (t,e) or -1;
 * slot_w[t,e] = its weight or 0.  Every row count is a multiple of M, so the
 * grouped GEMM runs whole tiles when M is its tile height (256).
 * At most moe_token_round_max_rows(T,E,K,M) = min(T*E, T*K + E*floor(M/2))
 * rows; the size functions return 0 for invalid sizes.  1 <= M <= 65536,
 * T*E < 2^31.
 */
long long moe_token_round_max_rows(int T, int E, int K, int M);
size_t moe_token_round_workspace_bytes(int T, int E, int K, int M);

/*
 * moe_token_round -- the plan from router logits and moe_route's routing.
 * In:  logits [T,E] fp32, topk_idx [T,K] int32 and counts [E] int32 as
 *      moe_route writes them (counts must be the histogram of topk_idx;
 *      otherwise the plan is unspecified, but nothing is written past
 *      rows_cap rows).
 * Out: counts_r [E], offsets_r [E+1], row_tok [rows_cap] (the first
 *      offsets_r[E] entries are written), slot_row [T,E] int32, slot_w [T,E]
 *      fp32.  rows_cap must be at least moe_token_round_max_rows(T,E,K,M).
 * Workspace: moe_token_round_workspace_bytes(T,E,K,M) bytes.
 */
int moe_token_round(const float* logits, const int32_t* topk_idx, const int32_t* counts, int T, int E, int K,
                    int M, int cap_tiles, int32_t* counts_r, int32_t* offsets_r, int32_t* row_tok,
                    long long rows_cap, int32_t* slot_row, float* slot_w, void* ws, size_t ws_bytes,
                    void* stream);

/*
 * moe_tr_combine -- step 5 after Token Rounding: a gather-sum by token over
 * the experts it kept, in ascending expert order, no atomics:
 *   out[t] = sum_{e: 0 <= slot_row[t,e] < rows} slot_w[t,e] * Y[slot_row[t,e]]
 * in fp32, rounded once to dtype (a token with no row gets zeros).
 * In:  Y [rows,d] (dtype), slot_row [T,E] int32, slot_w [T,E] fp32.
 * Out: out [T,d] (dtype).
 */
int moe_tr_combine(const void* Y, const int32_t* slot_row, const float* slot_w, int dtype, int T, int E, int d,
                   long long rows, void* out, void* stream);

/*
 * moe_forward_tr -- the whole layer with Token Rounding: moe_route,
 * moe_token_round, the grouped SwiGLU and down GEMMs over the plan's rows
 * (gathering X rows through row_tok where the tile kernel can) and
 * moe_tr_combine, on one stream.
 * In:  as moe_forward, plus M and cap_tiles.  Out: out [T,d].
 * Optional outputs (may be NULL, then they live in the workspace):
 *      counts_r [E], offsets_r [E+1], row_tok [moe_token_round_max_rows],
 *      slot_row [T,E], slot_w [T,E].
 * Workspace: moe_forward_tr_workspace_bytes(T,d,E,K,n,M,dtype) bytes.
 */
size_t moe_forward_tr_workspace_bytes(int T, int d, int E, int K, int n, int M, int dtype);
int moe_forward_tr(const void* X, const float* logits, const void* W1, const void* W3, const void* W2, int dtype,
                   int T, int d, int E, int K, int n, int M, int cap_tiles, void* out, int32_t* counts_r,
                   int32_t* offsets_r, int32_t* row_tok, int32_t* slot_row, float* slot_w, void* ws,
                   size_t ws_bytes, void* stream);

/*
 * moe_backward_data -- the data gradients of the layer that moe_forward
 * computes: dX and the router-logit gradient, given dout = dL/d(out).
 * [P4] section 2.2 names the backward's dH (through the SwiGLU) and dS (the
 * routing-score gradient, taken as <dA, A> so that the expert outputs need
 * not be kept); section 5 measures the backward.  Per assignment (t, k) with
 * expert e and weight w_k (moe_route's routing of `logits`), g = dout[t]:
 *   dA = g W2[e]^T, a = SiLU(h1) h3 with h1 = x W1[e], h3 = x W3[e] recomputed,
 *   dw[t,k] = <dA, a>, dh1 = w_k dA h3 SiLU'(h1), dh3 = w_k dA SiLU(h1),
 *   dX[t] = sum_k dh1 W1[e]^T + dh3 W3[e]^T,
 *   dlogits[t, idx_k] = w_k (dw[t,k] - sum_j w_j dw[t,j]), 0 for other experts.
 * The expert-weight gradients are not computed here (moe_backward adds them).
 * In:  X [T,d], W1/W3 [E,d,n], W2 [E,n,d] and dout [T,d] in dtype; logits
 *      [T,E] fp32.  Sizes and limits as moe_forward.
 * Out: dX [T,d] (dtype), dlogits [T,E] fp32, dw [T,K] fp32 (may be NULL).
 *      bf16 intermediates (h1, h3, dA, dh) are rounded to bf16 (dA in
 *      registers: the SwiGLU backward and dS run in the epilogue of the GEMM
 *      that forms it); the sums are fp32.
 * Workspace: moe_backward_data_workspace_bytes(T,d,E,K,n,dtype) bytes, 16-byte
 *      aligned; it holds the routing, expert-sorted copies of X and dout and
 *      the intermediates, all rewritten on every call.  For fp32, or for bf16
 *      with n or d not a multiple of 256, it also holds transposed copies of
 *      the weights (the bf16 GEMM otherwise reads them as stored).  The caller owns every buffer.  Errors as moe_forward:
 *      nothing is launched when an argument is rejected.
 */
size_t moe_backward_data_workspace_bytes(int T, int d, int E, int K, int n, int dtype);
int moe_backward_data(const void* X, const float* logits, const void* W1, const void* W3, const void* W2, int dtype,
                      int T, int d, int E, int K, int n, const void* dout, void* dX, float* dlogits, float* dw,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * moe_backward -- moe_backward_data plus the expert-weight gradients, summed
 * over the assignments of each expert (in ascending row order, fp32):
 *   dW1[e] = sum x^T dh1,  dW3[e] = sum x^T dh3,  dW2[e] = sum (w_k a)^T g
 * with x the token row, dh1, dh3, a and g as in moe_backward_data.
 * Out: as moe_backward_data, plus dW1, dW3 [E,d,n] and dW2 [E,n,d] fp32
 *      (required, 16-byte aligned; experts with no rows get zeros).
 * Workspace: moe_backward_workspace_bytes(T,d,E,K,n,dtype) bytes (the data
 *      backward's plus one [T*K, n] buffer).  Errors as moe_backward_data.
 */
size_t moe_backward_workspace_bytes(int T, int d, int E, int K, int n, int dtype);
int moe_backward(const void* X, const float* logits, const void* W1, const void* W3, const void* W2, int dtype, int T,
                 int d, int E, int K, int n, const void* dout, void* dX, float* dlogits, float* dw, float* dW1,
                 float* dW3, float* dW2, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
