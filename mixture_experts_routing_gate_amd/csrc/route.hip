// Steps 1-2 of the MoE layer forward: the fused softmax top-K gate with an LDS
// histogram per token chunk, and the scan that turns chunk histograms into
// per-expert counts, exclusive offsets and per-chunk placement bases.
//
// Gate semantics follow page [P1] "Optimising MoE with Triton: topk_gating
// operator fusion in practice" section 1 (softmax over the expert axis, then
// top-k, then a per-expert accumulation) fused as in its section 2.1 (softmax
// values stay in registers and feed the top-k directly; candidates are
// exchanged across lanes), and page [P4] "MoE architecture optimisation and
// SonicMoE practice" section 1 (the K best of E scores per token) and section
// 3.1 (per-expert counts).  The kernel design is gfx950's own: a group of G
// lanes owns one token row, 8 logits per lane, so E <= 8*G.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

// ---------------------------------------------------------------------------
// Gate.  A group of G adjacent lanes owns one token row, V logits per lane
// (lane g of the group holds experts g*V .. g*V+V-1), so E <= V*G.
//
// Fast path (value-only selection network).  Each logit becomes a 32-bit key
// that orders like the float: the order-preserving integer image of the
// (sign-canonicalised) fp32 value with its IB low bits replaced by
// (2^IB - 1 - e), IB = log2(V*G).  Larger key = larger logit, and between
// equal-looking keys the lower expert wins.  Top-KP keys per lane come from
// min/max sorting networks and bitonic merges; DPP exchanges merge the lane
// lists of a group.  The expert index and the slot order are read straight
// off the sorted keys.
//
// Exactness.  Dropping IB mantissa bits can only misorder logits whose keys
// share the upper 32-IB bits.  The fast result is therefore accepted only if
// no two of the K chosen keys share that prefix and exactly one key of the
// whole row has the prefix of the K-th chosen key; otherwise (exact ties,
// near-ties) the row is redone by the exact path: K rounds of a group-wide
// argmax on the fp32 logits, largest first, lower index among equal values.
//
// Weights use the exact logits of the chosen experts (re-read from cache):
// w_k = exp(l_k - l_0) / sum_j exp(l_j - l_0), the softmax renormalised over
// the K chosen experts.
// ---------------------------------------------------------------------------

MOE_DEV void cswap_desc(uint32_t& a, uint32_t& b) {
    const uint32_t hi = max(a, b), lo = min(a, b);
    a = hi;
    b = lo;
}

// Sorting networks (descending) for N in {1, 2, 4, 8}: Batcher odd-even merge.
template <int N>
MOE_DEV void sort_desc(uint32_t* a) {
    if constexpr (N == 2) {
        cswap_desc(a[0], a[1]);
    } else if constexpr (N == 4) {
        cswap_desc(a[0], a[1]); cswap_desc(a[2], a[3]);
        cswap_desc(a[0], a[2]); cswap_desc(a[1], a[3]);
        cswap_desc(a[1], a[2]);
    } else if constexpr (N == 8) {
        cswap_desc(a[0], a[1]); cswap_desc(a[2], a[3]); cswap_desc(a[4], a[5]); cswap_desc(a[6], a[7]);
        cswap_desc(a[0], a[2]); cswap_desc(a[1], a[3]); cswap_desc(a[4], a[6]); cswap_desc(a[5], a[7]);
        cswap_desc(a[1], a[2]); cswap_desc(a[5], a[6]);
        cswap_desc(a[0], a[4]); cswap_desc(a[1], a[5]); cswap_desc(a[2], a[6]); cswap_desc(a[3], a[7]);
        cswap_desc(a[2], a[4]); cswap_desc(a[3], a[5]);
        cswap_desc(a[1], a[2]); cswap_desc(a[3], a[4]); cswap_desc(a[5], a[6]);
    }
}

// a <- top N of (a union b); both sorted descending.  max(a_i, b_{N-1-i}) is a
// bitonic sequence holding the top N; a half-cleaner cascade sorts it.
template <int N>
MOE_DEV void merge_top(uint32_t* a, const uint32_t* b) {
#pragma unroll
    for (int i = 0; i < N; ++i) a[i] = max(a[i], b[N - 1 - i]);
#pragma unroll
    for (int s = N / 2; s >= 1; s /= 2)
#pragma unroll
        for (int i = 0; i < N; ++i)
            if ((i & s) == 0) cswap_desc(a[i], a[i + s]);
}

// Cross-lane exchange partners for the merge levels of a group (within a
// 16-lane DPP row): quad xor 1, quad xor 2, half-row mirror.
template <int LEVEL>
MOE_DEV uint32_t dpp_partner(uint32_t x) {
    constexpr int ctrl = LEVEL == 0 ? 0xB1 : LEVEL == 1 ? 0x4E : 0x141;
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, ctrl, 0xF, 0xF, false);
}
template <int LEVEL>
MOE_DEV float dpp_partner_f(float x) {
    return __builtin_bit_cast(float, dpp_partner<LEVEL>(__builtin_bit_cast(uint32_t, x)));
}

// Order-preserving integer image of a float (after -0.0 -> +0.0).
MOE_DEV uint32_t ord_key(float x) {
    const uint32_t u = __float_as_uint(x + 0.0f);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Exact selection for the rows of one wave whose fast result was rejected
// (`mine`): K rounds of a group-wide argmax on the fp32 logits, largest first,
// lower expert index among equal values (-0.0 == +0.0).  All lanes of the wave
// take part in the cross-lane reductions; only `mine` lanes write.
template <int V, int G>
__device__ __attribute__((noinline)) void gate_exact_rows(const float* lrow, bool mine, int t, int E, int K, int g,
                                                          int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_w, int* hist) {
    float v[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int e = g * V + j;
        const float x = lrow[e < E ? e : 0] + 0.0f;
        v[j] = (mine && e < E) ? x : -INFINITY;
    }
    float sv[8];
    int si[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        sv[r] = 0.0f;
        si[r] = 0;
        if (r < K) {
            float bv = v[0];
            int bj = 0;
#pragma unroll
            for (int j = 1; j < V; ++j)
                if (v[j] > bv) {
                    bv = v[j];
                    bj = j;
                }
            const float M = group_max<G>(bv);
            const int cand = (bv == M) ? g * V + bj : 0x7fffffff;
            const int I = group_min<G>(cand);
#pragma unroll
            for (int j = 0; j < V; ++j)
                if (g * V + j == I) v[j] = -INFINITY;
            sv[r] = M;
            si[r] = I;
        }
    }
    float exs[8];
    float ps = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        exs[r] = 0.0f;
        if (r < K && (r % G) == g) {
            exs[r] = expf(sv[r] - sv[0]);
            ps += exs[r];
        }
    }
    const float S2 = group_sum<G>(ps);
    if (mine) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if (r < K && (r % G) == g) {
                topk_idx[(size_t)t * K + r] = si[r];
                topk_w[(size_t)t * K + r] = exs[r] / S2;
                // only non-finite logits (outside the contract) leave si out of range
                if ((unsigned)si[r] < (unsigned)E) atomicAdd(&hist[si[r]], 1);
            }
        }
    }
}

template <int V, int G, int KP, int THREADS, bool VEC, bool PAD>
__global__ __launch_bounds__(THREADS) void gate_kernel(const float* __restrict__ logits, int T, int E,
                                                       int K, int CH, int32_t* __restrict__ topk_idx,
                                                       float* __restrict__ topk_w, int32_t* __restrict__ blk) {
    constexpr int RPW = kWave / G;                 // rows per wave per pass
    constexpr int RPB = RPW * (THREADS / kWave);   // rows per workgroup per pass
    constexpr int EP = V * G;                      // padded expert count (power of two)
    constexpr int IB = EP <= 8 ? 3 : EP <= 16 ? 4 : EP <= 32 ? 5 : EP <= 64 ? 6 : EP <= 128 ? 7 : 8;
    constexpr uint32_t IMASK = (1u << IB) - 1u;
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
    static_assert(V % KP == 0 && V % 4 == 0, "lane width");
    __shared__ int hist[256];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int g = lane % G;
    const int rw = lane / G;
    for (int e = tid; e < E; e += THREADS) hist[e] = 0;
    __syncthreads();

    const int chunk = blockIdx.x;
    const int t0 = chunk * CH;
    const int t1 = min(T, t0 + CH);
    for (int base = t0 + wave * RPW; base < t1; base += RPB) {
        const int t = base + rw;
        const bool valid = t < t1;
        // ---- keys ----
        // Loads are unconditional (row and column clamped into the tensor) so
        // that all of a lane's loads are in flight together; padding columns
        // get key 0 (below every logit).  Rows past the chunk are computed and
        // discarded: nothing of theirs is stored or counted.
        const float* lrow = logits + (size_t)min(t, T - 1) * E;
        // index bits IMASK - e; V is a power of two, so IMASK - g*V - j == (IMASK - g*V) ^ j
        const uint32_t ibase = IMASK - (uint32_t)(g * V);
        uint32_t key[V];
        if constexpr (VEC) {
            f32x4 x[V / 4];
#pragma unroll
            for (int q = 0; q < V / 4; ++q) {
                const int e0 = g * V + q * 4;
                x[q] = *reinterpret_cast<const f32x4*>(lrow + (e0 < E ? e0 : 0));
            }
#pragma unroll
            for (int q = 0; q < V / 4; ++q) {
                const bool ok = !PAD || (g * V + q * 4) < E;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t k = (ord_key(x[q][j]) & ~IMASK) | (ibase ^ (uint32_t)(q * 4 + j));
                    key[q * 4 + j] = ok ? k : 0u;
                }
            }
        } else {
            float x[V];
#pragma unroll
            for (int j = 0; j < V; ++j) {
                const int e = g * V + j;
                x[j] = lrow[e < E ? e : 0];
            }
#pragma unroll
            for (int j = 0; j < V; ++j) {
                const bool ok = !PAD || (g * V + j) < E;
                const uint32_t k = (ord_key(x[j]) & ~IMASK) | (ibase ^ (uint32_t)j);
                key[j] = ok ? k : 0u;
            }
        }

        // ---- top-KP keys of the lane ----
        uint32_t top[KP];
#pragma unroll
        for (int i = 0; i < KP; ++i) top[i] = key[i];
        sort_desc<KP>(top);
#pragma unroll
        for (int c = 1; c < V / KP; ++c) {
            uint32_t nxt[KP];
#pragma unroll
            for (int i = 0; i < KP; ++i) nxt[i] = key[c * KP + i];
            sort_desc<KP>(nxt);
            merge_top<KP>(top, nxt);
        }
        // ---- merge across the G lanes of the row ----
        if constexpr (G >= 2) {
            uint32_t o[KP];
#pragma unroll
            for (int i = 0; i < KP; ++i) o[i] = dpp_partner<0>(top[i]);
            merge_top<KP>(top, o);
        }
        if constexpr (G >= 4) {
            uint32_t o[KP];
#pragma unroll
            for (int i = 0; i < KP; ++i) o[i] = dpp_partner<1>(top[i]);
            merge_top<KP>(top, o);
        }
        if constexpr (G >= 8) {
            uint32_t o[KP];
#pragma unroll
            for (int i = 0; i < KP; ++i) o[i] = dpp_partner<2>(top[i]);
            merge_top<KP>(top, o);
        }

        // ---- exactness check ----
        uint32_t kth = top[0];
        bool dup = false;
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            if (i + 1 < KP && i + 1 < K) dup |= (top[i] >> IB) == (top[i + 1] >> IB);
            if (i == K - 1) kth = top[i];
        }
        // keys whose prefix is >= the K-th key's prefix: exactly K unless some
        // unchosen logit shares the K-th one's prefix (internal ones are in dup)
        const uint32_t thr = kth & ~IMASK;
        int same = 0;
#pragma unroll
        for (int j = 0; j < V; ++j) same += (key[j] >= thr) ? 1 : 0;
        if constexpr (G >= 2) same += (int)dpp_partner<0>((uint32_t)same);
        if constexpr (G >= 4) same += (int)dpp_partner<1>((uint32_t)same);
        if constexpr (G >= 8) same += (int)dpp_partner<2>((uint32_t)same);
        const bool exact_fast = !dup && same == K;

        // ---- weights and outputs of accepted rows ----
        // Lane g of the group owns slots r = g + G*i.  Its slot keys are picked
        // from the group-uniform list with a static select chain (no divergent
        // branches), and the exact logits of all its slots are loaded together.
        constexpr int SPL = (KP + G - 1) / G;  // slots per lane
        uint32_t mk[SPL];
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            mk[i] = top[0];
#pragma unroll
            for (int gg = 0; gg < G; ++gg)
                if (gg + G * i < KP && g == gg) mk[i] = top[gg + G * i];
        }
        const int e0 = min((int)(IMASK - (top[0] & IMASK)), E - 1);
        int er[SPL];
        float xr[SPL];
#pragma unroll
        for (int i = 0; i < SPL; ++i) er[i] = min((int)(IMASK - (mk[i] & IMASK)), E - 1);
        const float l0 = lrow[e0];
#pragma unroll
        for (int i = 0; i < SPL; ++i) xr[i] = lrow[er[i]];
        float ex[SPL];
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            const bool act = g + G * i < K;
            ex[i] = act ? expf(xr[i] - l0) : 0.0f;
            part += ex[i];
        }
        float S = part;
        if constexpr (G >= 2) S += dpp_partner_f<0>(S);
        if constexpr (G >= 4) S += dpp_partner_f<1>(S);
        if constexpr (G >= 8) S += dpp_partner_f<2>(S);
        if (valid && exact_fast) {
#pragma unroll
            for (int i = 0; i < SPL; ++i) {
                const int r = g + G * i;
                if (r < K) {
                    topk_idx[(size_t)t * K + r] = er[i];
                    topk_w[(size_t)t * K + r] = ex[i] / S;
                    atomicAdd(&hist[er[i]], 1);
                }
            }
        }

        // ---- exact path for rows with (near-)ties ----
        if (__builtin_amdgcn_ballot_w64(valid && !exact_fast) != 0)
            gate_exact_rows<V, G>(lrow, valid && !exact_fast, t, E, K, g, topk_idx, topk_w, hist);
    }
    __syncthreads();
    for (int e = tid; e < E; e += THREADS) blk[(size_t)chunk * E + e] = hist[e];
}

// One workgroup of 1024 threads.  blk is [B, E] (per-chunk counts).  Produces
// counts[e] = sum_b blk[b,e], offsets = exclusive scan of counts with
// offsets[E] = total, and (if blkbase != nullptr) the placement base of every
// chunk: blkbase[b,e] = offsets[e] + sum_{b' < b} blk[b',e].
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void scan_kernel(const int32_t* __restrict__ blk, int B,
                                                            int E, int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ blkbase) {
    __shared__ int part[kScanThreads];  // [Q][E]: chunk-group sums, then their exclusive prefix
    __shared__ int sc[2][256];          // scan buffers over experts
    const int tid = threadIdx.x;
    const int Q = kScanThreads / E;  // chunk groups (>= 4 since E <= 256)
    const int e = tid % E;
    const int q = tid / E;
    const bool act = q < Q;
    const int b0 = act ? (int)(((long long)B * q) / Q) : 0;
    const int b1 = act ? (int)(((long long)B * (q + 1)) / Q) : 0;
    if (act) {
        // batches of 8 independent loads keep the latency of the strided reads overlapped
        int s = 0;
        int b = b0;
        for (; b + 8 <= b1; b += 8) {
            int x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = blk[(size_t)(b + i) * E + e];
#pragma unroll
            for (int i = 0; i < 8; ++i) s += x[i];
        }
        for (; b < b1; ++b) s += blk[(size_t)b * E + e];
        part[tid] = s;
    }
    __syncthreads();
    if (tid < E) {
        int run = 0;
        for (int qq = 0; qq < Q; ++qq) {
            const int x = part[qq * E + tid];
            part[qq * E + tid] = run;
            run += x;
        }
        counts[tid] = run;
        sc[0][tid] = run;
    } else if (tid < 256) {
        sc[0][tid] = 0;
    }
    __syncthreads();
    int cur = 0;
    for (int sh = 1; sh < 256; sh <<= 1) {  // inclusive scan over experts
        int x = 0;
        if (tid < 256) {
            x = sc[cur][tid];
            if (tid >= sh) x += sc[cur][tid - sh];
        }
        __syncthreads();
        if (tid < 256) sc[cur ^ 1][tid] = x;
        __syncthreads();
        cur ^= 1;
    }
    if (tid < E) {
        offsets[tid] = (tid == 0) ? 0 : sc[cur][tid - 1];
        if (tid == E - 1) offsets[E] = sc[cur][tid];
    }
    if (blkbase != nullptr && act) {
        int run = (e == 0 ? 0 : sc[cur][e - 1]) + part[q * E + e];
        int b = b0;
        for (; b + 8 <= b1; b += 8) {
            int x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = blk[(size_t)(b + i) * E + e];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                blkbase[(size_t)(b + i) * E + e] = run;
                run += x[i];
            }
        }
        for (; b < b1; ++b) {
            blkbase[(size_t)b * E + e] = run;
            run += blk[(size_t)b * E + e];
        }
    }
}

template <int V, int G, int KP>
hipError_t launch_gate_v(const float* logits, int T, int E, int K, int32_t* idx, float* w,
                         int32_t* blk, hipStream_t s) {
    constexpr int THREADS = G >= 4 ? 1024 : 256 * G;
    const dim3 grid(num_chunks(T));
    const int CH = chunk_tokens(T);
    if (E == V * G)  // no padding columns; E is then a multiple of 4
        hipLaunchKernelGGL((gate_kernel<V, G, KP, THREADS, true, false>), grid, dim3(THREADS), 0, s, logits, T,
                           E, K, CH, idx, w, blk);
    else if ((E & 3) == 0)
        hipLaunchKernelGGL((gate_kernel<V, G, KP, THREADS, true, true>), grid, dim3(THREADS), 0, s, logits, T, E,
                           K, CH, idx, w, blk);
    else
        hipLaunchKernelGGL((gate_kernel<V, G, KP, THREADS, false, true>), grid, dim3(THREADS), 0, s, logits, T,
                           E, K, CH, idx, w, blk);
    return hipGetLastError();
}

template <int V, int G>
hipError_t launch_gate_k(const float* logits, int T, int E, int K, int32_t* idx, float* w,
                         int32_t* blk, hipStream_t s) {
    if (K <= 1) return launch_gate_v<V, G, 1>(logits, T, E, K, idx, w, blk, s);
    if (K <= 2) return launch_gate_v<V, G, 2>(logits, T, E, K, idx, w, blk, s);
    if (K <= 4) return launch_gate_v<V, G, 4>(logits, T, E, K, idx, w, blk, s);
    return launch_gate_v<V, G, 8>(logits, T, E, K, idx, w, blk, s);
}

}  // namespace

hipError_t launch_gate(const float* logits, int T, int E, int K, int32_t* idx, float* w,
                       int32_t* blk, hipStream_t s) {
    if (E <= 8) return launch_gate_k<8, 1>(logits, T, E, K, idx, w, blk, s);
    if (E <= 32) return launch_gate_k<32, 1>(logits, T, E, K, idx, w, blk, s);
    if (E <= 64) return launch_gate_k<32, 2>(logits, T, E, K, idx, w, blk, s);
    if (E <= 128) return launch_gate_k<32, 4>(logits, T, E, K, idx, w, blk, s);
    return launch_gate_k<32, 8>(logits, T, E, K, idx, w, blk, s);
}

hipError_t launch_scan(const int32_t* blk, int B, int E, int32_t* counts, int32_t* offsets,
                       int32_t* blkbase, hipStream_t s) {
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, blk, B, E, counts, offsets,
                       blkbase);
    return hipGetLastError();
}

}  // namespace moe
