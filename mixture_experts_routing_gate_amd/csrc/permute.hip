// Step 3 of the MoE layer forward: token rows into expert-contiguous order.
//
// Page [P2] "SpMM in MoE: accelerating sparse experts with Triton kernels"
// section 6 repeats each token row once per selected expert; page [P4] "MoE
// architecture optimisation and SonicMoE practice" section 1 (gather) and
// section 2.2 (intermediates stored grouped by expert).  The order is a stable
// counting sort of the row-major (token, slot) list by expert, so it is unique
// and reproducible: rank(t,k) = chunk base + rows of the same expert earlier in
// the chunk.  Ranks inside a chunk use per-wave 64-bit lane masks built with
// LDS integer ORs (commutative, hence deterministic) and popcounts.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// Per-chunk expert histogram of topk_idx (entries outside [0,E) are ignored).
__global__ __launch_bounds__(kThreads) void chunk_hist_kernel(const int32_t* __restrict__ idx, int T,
                                                              int E, int K, int CH,
                                                              int32_t* __restrict__ blk) {
    __shared__ int hist[256];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kThreads) hist[e] = 0;
    __syncthreads();
    const size_t q0 = (size_t)blockIdx.x * CH * K;
    const size_t q1 = (size_t)min(T, (int)(blockIdx.x + 1) * CH) * K;
    for (size_t q = q0 + tid; q < q1; q += kThreads) {
        const int e = idx[q];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += kThreads) blk[(size_t)blockIdx.x * E + e] = hist[e];
}

// One workgroup per chunk.  Tokens are taken 256 at a time (one per thread);
// wave w sets bit `lane` of mask[w][e] for each expert e its token selected.
// Position of (t,k) = base(chunk,e) + earlier sub-chunks + earlier waves +
// popcount(mask[w][e] & lanes below).
//
// The counts may be kept per sub-chunk: `sub` rows of blk (or blkbase) per
// chunk of CH tokens (the fused router-gate counts 32-token tiles).
// base(chunk,e) comes from blkbase (its row chunk*sub) when it is given.
// Otherwise (small B*E) every workgroup does the scan of step 2 itself from
// the counts blk[B,E]: thread e adds expert e over all B rows (its count) and
// over the rows before this chunk's first, then an exclusive scan over experts
// gives offsets.  Workgroup 0 writes counts and offsets when they are not
// null.  The sums are of integers, so every workgroup gets the same values in
// any order.
__global__ __launch_bounds__(kThreads) void rank_kernel(const int32_t* __restrict__ idx, int T, int E,
                                                        int K, int CH, int sub,
                                                        const int32_t* __restrict__ blkbase,
                                                        const int32_t* __restrict__ blk, int B,
                                                        int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ sorted_pair,
                                                        int32_t* __restrict__ inv,
                                                        int* __restrict__ zero, int nzero) {
    __shared__ unsigned long long mask[kWaves][256];
    __shared__ int pre[kWaves][256];
    __shared__ int run[256];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int chunk = blockIdx.x;
    if (chunk == 0)  // state for later kernels on the stream
        for (int i = tid; i < nzero; i += kThreads) zero[i] = 0;
    if (blkbase != nullptr) {
        for (int e = tid; e < E; e += kThreads) run[e] = blkbase[(size_t)chunk * sub * E + e];
    } else {  // E <= 256 == kThreads: thread e owns expert e
        constexpr int kBatch = 16;
        int tot = 0, below = 0;
        if (tid < E) {
            for (int b0 = 0; b0 < B; b0 += kBatch) {
                int x[kBatch];
#pragma unroll
                for (int i = 0; i < kBatch; ++i) x[i] = blk[(size_t)min(b0 + i, B - 1) * E + tid];
#pragma unroll
                for (int i = 0; i < kBatch; ++i) {
                    const int v = (b0 + i < B) ? x[i] : 0;
                    tot += v;
                    below += (b0 + i < chunk * sub) ? v : 0;
                }
            }
        }
        int* sc0 = pre[0];
        int* sc1 = pre[1];
        sc0[tid] = tot;
        __syncthreads();
        for (int sh = 1; sh < 256; sh <<= 1) {  // inclusive scan over experts
            const int x = sc0[tid] + (tid >= sh ? sc0[tid - sh] : 0);
            __syncthreads();
            sc1[tid] = x;
            __syncthreads();
            int* t = sc0;
            sc0 = sc1;
            sc1 = t;
        }
        if (tid < E) {
            const int excl = sc0[tid] - tot;
            run[tid] = excl + below;
            if (chunk == 0 && counts != nullptr) counts[tid] = tot;
            if (chunk == 0 && offsets != nullptr) {
                offsets[tid] = excl;
                if (tid == E - 1) offsets[E] = sc0[tid];
            }
        }
    }
    for (int e = tid; e < E; e += kThreads) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) mask[w][e] = 0ull;
    }
    __syncthreads();
    const int t0 = chunk * CH;
    const int t1 = min(T, t0 + CH);
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int sub = t0; sub < t1; sub += kThreads) {
        const int t = sub + tid;
        const bool valid = t < t1;
        int ek[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            ek[k] = -1;
            if (k < K && valid) {
                const int e = idx[(size_t)t * K + k];
                if (e >= 0 && e < E) {
                    ek[k] = e;
                    atomicOr(&mask[wave][e], 1ull << lane);
                }
            }
        }
        __syncthreads();
        for (int e = tid; e < E; e += kThreads) {
            int r = run[e];
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                pre[w][e] = r;
                r += __popcll(mask[w][e]);
            }
            run[e] = r;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int e = ek[k];
            if (e >= 0) {
                const int pos = pre[wave][e] + __popcll(mask[wave][e] & below);
                sorted_pair[pos] = t * K + k;
                inv[(size_t)t * K + k] = pos;
            }
        }
        __syncthreads();
        for (int e = tid; e < E; e += kThreads) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) mask[w][e] = 0ull;
        }
        __syncthreads();
    }
}

// One wave per token: read the row once (16-byte chunks, kUnroll per lane in
// flight), write it to its K expert-ordered positions.
constexpr int kCopyUnroll = 8;

__global__ __launch_bounds__(kThreads) void copy_rows_kernel(const u32x4* __restrict__ X, int T,
                                                             int row_chunks, int K,
                                                             const int32_t* __restrict__ inv,
                                                             u32x4* __restrict__ Xp) {
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * kWaves + threadIdx.x / kWave;
    if (t >= T) return;
    const int A = T * K;
    int pos[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        pos[k] = (k < K) ? uniform(inv[(size_t)t * K + k]) : -1;
        if ((unsigned)pos[k] >= (unsigned)A) pos[k] = -1;  // never write outside Xp, whatever inv holds
    }
    const u32x4* src = X + (size_t)t * row_chunks;
    for (int c0 = 0; c0 < row_chunks; c0 += kWave * kCopyUnroll) {
        u32x4 buf[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int c = c0 + u * kWave + lane;
            if (c < row_chunks) buf[u] = __builtin_nontemporal_load(src + c);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (k < K && pos[k] >= 0) {
                u32x4* dst = Xp + (size_t)pos[k] * row_chunks;
#pragma unroll
                for (int u = 0; u < kCopyUnroll; ++u) {
                    const int c = c0 + u * kWave + lane;
                    if (c < row_chunks) dst[c] = buf[u];
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_chunk_hist(const int32_t* idx, int T, int E, int K, int32_t* blk, hipStream_t s) {
    hipLaunchKernelGGL(chunk_hist_kernel, dim3(num_chunks(T)), dim3(kThreads), 0, s, idx, T, E, K,
                       chunk_tokens(T), blk);
    return hipGetLastError();
}

hipError_t launch_rank(const int32_t* idx, int T, int E, int K, const int32_t* blkbase,
                       int32_t* sorted_pair, int32_t* inv, hipStream_t s, int sub_tokens) {
    const int ST = sub_tokens > 0 ? sub_tokens : chunk_tokens(T);
    hipLaunchKernelGGL(rank_kernel, dim3(num_chunks(T)), dim3(kThreads), 0, s, idx, T, E, K,
                       chunk_tokens(T), chunk_tokens(T) / ST, blkbase, static_cast<const int32_t*>(nullptr), 0,
                       static_cast<int32_t*>(nullptr), static_cast<int32_t*>(nullptr), sorted_pair, inv,
                       static_cast<int*>(nullptr), 0);
    return hipGetLastError();
}

hipError_t launch_scan_rank(const int32_t* idx, int T, int E, int K, const int32_t* blk, int32_t* counts,
                            int32_t* offsets, int32_t* sorted_pair, int32_t* inv, int* zero, int nzero,
                            hipStream_t s, int sub_tokens) {
    const int ST = sub_tokens > 0 ? sub_tokens : chunk_tokens(T);
    hipLaunchKernelGGL(rank_kernel, dim3(num_chunks(T)), dim3(kThreads), 0, s, idx, T, E, K,
                       chunk_tokens(T), chunk_tokens(T) / ST, static_cast<const int32_t*>(nullptr), blk,
                       (T + ST - 1) / ST, counts, offsets, sorted_pair, inv, zero, zero != nullptr ? nzero : 0);
    return hipGetLastError();
}

hipError_t launch_copy_rows(const void* X, size_t row_bytes, int T, int K, const int32_t* inv,
                            void* Xp, hipStream_t s) {
    const int row_chunks = (int)(row_bytes / 16);
    hipLaunchKernelGGL(copy_rows_kernel, dim3((T + kWaves - 1) / kWaves), dim3(kThreads), 0, s,
                       static_cast<const u32x4*>(X), T, row_chunks, K, inv, static_cast<u32x4*>(Xp));
    return hipGetLastError();
}

}  // namespace moe
