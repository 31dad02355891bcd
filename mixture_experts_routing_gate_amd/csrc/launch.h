// Host-side launchers of the libmoe kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Tokens per chunk: the gate writes one expert histogram per chunk and the
// permutation places each chunk's rows at that chunk's base, so the stable
// order needs no cross-chunk communication beyond one scan.
inline int chunk_tokens(int T) { return T <= 65536 ? 256 : 1024; }
inline int num_chunks(int T) { return (T + chunk_tokens(T) - 1) / chunk_tokens(T); }

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Steps 1-2.
hipError_t launch_gate(const float* logits, int T, int E, int K, int32_t* idx, float* w,
                       int32_t* blk, hipStream_t s);
// `zero` (nullable): nzero ints the scan also clears (state for later kernels
// on the stream, such as the grouped GEMMs' claim counters).
hipError_t launch_scan(const int32_t* blk, int B, int E, int32_t* counts, int32_t* offsets,
                       int32_t* blkbase, hipStream_t s, int* zero = nullptr, int nzero = 0);

// Step 3.
hipError_t launch_chunk_hist(const int32_t* idx, int T, int E, int K, int32_t* blk, hipStream_t s);
// sub_tokens (0 = chunk_tokens(T)): the token count of one row of blk /
// blkbase, a divisor of chunk_tokens(T) (the fused router-gate keeps counts
// per 32-token tile: kRouterGateTokens).
hipError_t launch_rank(const int32_t* idx, int T, int E, int K, const int32_t* blkbase,
                       int32_t* sorted_pair, int32_t* inv, hipStream_t s, int sub_tokens = 0);
// Scan and rank in one launch: each rank workgroup scans blk[B,E] itself
// (worth it while B*E is small, see scan_rank_fused()); counts and offsets are
// written when not null.
hipError_t launch_scan_rank(const int32_t* idx, int T, int E, int K, const int32_t* blk, int32_t* counts,
                            int32_t* offsets, int32_t* sorted_pair, int32_t* inv, int* zero, int nzero,
                            hipStream_t s, int sub_tokens = 0);
inline int count_rows(int T, int sub_tokens) {
    const int st = sub_tokens > 0 ? sub_tokens : chunk_tokens(T);
    return (T + st - 1) / st;
}
inline bool scan_rank_fused(int T, int E, int sub_tokens = 0) {
    return (long long)count_rows(T, sub_tokens) * E <= 16384;
}
hipError_t launch_copy_rows(const void* X, size_t row_bytes, int T, int K, const int32_t* inv,
                            void* Xp, hipStream_t s);

// Step 4.  dtype: 0 = fp32, 1 = bf16.  4a (SwiGLU GEMM), 4b (down GEMM), both.
// `part` (nullable) is the split workspace of ffn_split_bytes() bytes: with it,
// the last partial round of tiles is split over the idle workgroups along K,
// and tiles are claimed from per-XCD counters kept at its end
// (ffn_ticket_ints() ints at ffn_tickets(part)).  They must be zero when a GEMM
// starts: each launch clears its own set first unless `tickets_zeroed` says an
// earlier kernel on the stream already did.
size_t ffn_split_bytes(int dtype, int d, int n);
int* ffn_tickets(float* part);
int ffn_ticket_ints();
hipError_t launch_ffn_up(const void* Xp, const void* W1, const void* W3, int dtype, int rows, int d, int E,
                         int n, const int32_t* counts, const int32_t* offsets, void* Act, float* part,
                         bool tickets_zeroed, hipStream_t s, const int32_t* gather = nullptr, int gK = 1,
                         int xrows = 0);
// H1 = Xp W1 into H and H3 = Xp W3 into H + rows * n, bf16, one launch (needs
// the pipelined kernel's sizes: ffn_raw_ok(1, d, n)).
bool ffn_raw_ok(int dtype, int d, int n);
hipError_t launch_ffn_up_raw(const void* Xp, const void* W1, const void* W3, int rows, int d, int E, int n,
                             const int32_t* counts, const int32_t* offsets, void* H, hipStream_t s);
hipError_t launch_ffn_down(const void* Act, const void* W2, int dtype, int rows, int d, int E, int n,
                           const int32_t* counts, const int32_t* offsets, void* Y, float* part,
                           bool tickets_zeroed, hipStream_t s);
// The router projection logits = X [hi ; lo] summed per column, plus bias, on
// the SwiGLU GEMM's kernel, where router_gemm_ok(T, d, E): bf16 X [T, d], hi
// and lo [d, E] bf16, counts = {T} and offsets = {0, T} in device memory, part
// the split workspace of ffn_split_bytes(1, d, E) bytes (its claim counters
// cleared first unless `tickets_zeroed`).  Deterministic.
bool router_gemm_ok(int T, int d, int E);
hipError_t launch_router_gemm(const uint16_t* X, const uint16_t* hi, const uint16_t* lo, int T, int d, int E,
                              const int32_t* counts, const int32_t* offsets, const float* bias, float* logits,
                              float* part, bool tickets_zeroed, hipStream_t s);
// C = A [B0^T ; B1^T] per expert (rows x N): B0 and B1 are each expert's
// N x kb row-major matrices, B1 only when Kd = 2 kb (nullptr when Kd = kb).
// bf16 pipelined kernel only: where ffn_bt_ok(), else hipErrorInvalidValue.
bool ffn_bt_ok(int dtype, int N, int Kd, int kb);
hipError_t launch_ffn_bt(const void* A, const void* B0, const void* B1, int kb, int dtype, int rows, int N, int E,
                         int Kd, const int32_t* counts, const int32_t* offsets, void* C, float* part,
                         bool tickets_zeroed, hipStream_t s);
// dA = A B0^T per expert (B0 [E, N, kb], k-contiguous, as launch_ffn_bt with
// Kd = kb) with the SwiGLU backward in the GEMM's epilogue: for each element,
// from H1, H3 [rows, N] and the row's routing weight wrow[rows], writes
// dH [rows, 2N] = [dh1 | dh3], aw [rows, N] = w * act (when not null) and one
// fp32 dS part per row and 64 columns, ds_part [rows, N / 64]; dA is not
// stored.  bf16, where ffn_bt_ok(1, N, kb, kb), else hipErrorInvalidValue.
hipError_t launch_ffn_bt_swiglu_bwd(const void* A, const void* B0, int kb, int rows, int N, int E,
                                    const int32_t* counts, const int32_t* offsets, const void* H1, const void* H3,
                                    void* dH, void* aw, const float* wrow, float* ds_part, hipStream_t s);
// Per expert-sorted row p: wrow[p] = topk_w[sorted_pair[p]]; and the dS of each
// row from its parts, added in part order: dS_tk[sorted_pair[p]] = sum_j ds_part[p, j].
hipError_t launch_row_weights(const float* topk_w, const int32_t* sorted_pair, int rows, float* wrow, hipStream_t s);
hipError_t launch_ds_reduce(const float* ds_part, int nparts, const int32_t* sorted_pair, int rows, float* dS_tk,
                            hipStream_t s);
// Expert-weight gradients on the pipelined kernel: dW[e] (M x N fp32) = sum over
// e's rows r of P[r, 0:M]^T Q[r, qoff:qoff+N]; bf16, where dw_p4_ok(), else
// hipErrorInvalidValue (rows = the total row count, for the offset range).
bool dw_p4_ok(int dtype, int E, int M, int N, int rows, int ldp, int ldq);
hipError_t launch_dw_p4(const void* P, int ldp, const void* Q, int ldq, int qoff, const int32_t* counts,
                        const int32_t* offsets, int E, int M, int N, int rows, float* dW, hipStream_t s);
hipError_t launch_ffn(const void* Xp, const void* W1, const void* W3, const void* W2, int dtype,
                      int rows, int d, int E, int n, const int32_t* counts, const int32_t* offsets,
                      void* Act, void* Y, float* part, bool tickets_zeroed, hipStream_t s,
                      const int32_t* gather = nullptr, int gK = 1, int xrows = 0);
// With `gather` the SwiGLU GEMM reads its rows straight from the token-ordered
// X (passed as Xp, xrows rows): row p of the expert-sorted order is X row
// gather[p] / gK, clamped into [0, xrows) (sorted_pair with gK = K, or a
// Token Rounding plan's row_tok with gK = 1).  Only where ffn_gather_ok().
bool ffn_gather_ok(int dtype, int T, int d, int n);

// Router projection upstream of step 1: logits = X Wr (+ bias).  `split` is a
// workspace of router_split_bytes() bytes (0: none needed) for the bf16 split
// of Wr.
size_t router_split_bytes(int dtype, int d, int E);
hipError_t launch_router(const void* X, int dtype, int T, int d, int E, const float* Wr, const float* bias,
                         float* logits, void* split, hipStream_t s);
// The router projection fused with the gate (steps 0-1 in one pass), where
// router_gate_ok(): bf16 X, d % 256 == 0, E <= 64.  Writes topk_idx, topk_w,
// the expert counts of each kRouterGateTokens-token tile into blk
// [ceil(T / kRouterGateTokens), E], and the logits when `logits` is not null.
// `split` as for launch_router.
constexpr int kRouterGateTokens = 32;
bool router_gate_ok(int dtype, int d, int E);
hipError_t launch_router_gate(const void* X, int T, int d, int E, int K, const float* Wr, const float* bias,
                              float* logits, int32_t* idx, float* w, int32_t* blk, void* split, hipStream_t s);

// Step 5.
hipError_t launch_combine(const void* Y, const float* w, const int32_t* inv, int dtype, int T, int d,
                          int K, void* out, hipStream_t s);

// Token Rounding (routing variant).  tr_target: rows kept by an expert with f
// routed tokens.  launch_token_round needs tr_keys_bytes(T, E) bytes of `ws`.
long long tr_target(int f, int M, int T, int cap_tiles);
size_t tr_keys_bytes(int T, int E);
hipError_t launch_token_round(const float* logits, const int32_t* idx, const int32_t* counts, int T, int E, int K,
                              int M, int cap_tiles, int32_t* counts_r, int32_t* offsets_r, int32_t* row_tok,
                              long long rows_cap, int32_t* slot_row, float* slot_w, void* ws, hipStream_t s);
hipError_t launch_tr_combine(const void* Y, const int32_t* slot_row, const float* slot_w, int dtype, int T, int E,
                             int d, long long nrows, void* out, hipStream_t s);
hipError_t launch_tr_gather_rows(const void* X, size_t row_bytes, int T, const int32_t* row_tok,
                                 const int32_t* offsets_r, int E, long long rows_cap, void* Xp, hipStream_t s);

// Backward, data gradients.  out[e*oes + c*ors + r] = in[e][r][c] for in
// [E][R][C] (dtype 0 fp32, 1 bf16); the SwiGLU backward with dS over
// expert-sorted rows; the router-logit gradient; a float fill.
hipError_t launch_transpose_experts(const void* in, int dtype, int E, int R, int C, void* out, size_t oes,
                                    size_t ors, hipStream_t s);
hipError_t launch_swiglu_bwd(const void* H1, const void* H3, const void* dA, const float* topk_w,
                             const int32_t* sorted_pair, int dtype, int rows, int n, void* dH, float* dS_tk,
                             void* aw, hipStream_t s);
// dW[e][m][c] = sum over expert e's rows r of P[r][m] Q[r][qoff + c] (fp32 out [E, M, N]);
// bf16 needs M and N multiples of 128.
hipError_t launch_dw(const void* P, int ldp, const void* Q, int ldq, int qoff, const int32_t* counts,
                     const int32_t* offsets, int dtype, int E, int M, int N, int rows, float* dW, hipStream_t s);
hipError_t launch_logit_grad(const int32_t* idx, const float* topk_w, const float* dS_tk, int T, int E, int K,
                             float* dlogits, hipStream_t s);
hipError_t launch_fill_f32(float* p, size_t n, float v, hipStream_t s);

}  // namespace moe
