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
// near-ties) the row is listed and, after the main loop, redone by the exact
// path: one wave per row, K rounds of a wave-wide argmax on the fp32 logits,
// largest first, lower index among equal values.
//
// Weights use the exact logits of the chosen experts (re-read from cache):
// w_k = exp(l_k - l_0) / sum_j exp(l_j - l_0), the softmax renormalised over
// the K chosen experts.
//
// Staging (E % 4 == 0).  Each wave owns an LDS region for the RPW rows of its
// pass.  The rows of the wave's next pass are copied into it by LDS-DMA as
// soon as the current ones have been read into registers, so the HBM reads of
// one pass overlap the selection work of the previous one.  The copy is
// 16-byte chunks, XOR-swizzled within each 1 KB so that the per-lane reads
// (lanes 128 bytes apart) spread over the LDS banks; rows past the chunk read
// as zeros (buffer bounds) and are discarded.
// ---------------------------------------------------------------------------

// Largest token chunk of one gate workgroup (chunk_tokens() never exceeds it).
constexpr int kMaxChunk = 1024;

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

// (v, i) <- the better of (v, i) and (ov, oi): larger value, then lower index.
MOE_DEV void argmax_take(float& v, int& i, float ov, int oi) {
    const bool take = (ov > v) | ((ov == v) & (oi < i));
    v = take ? ov : v;
    i = take ? oi : i;
}
template <int CTRL, int ROW_MASK>
MOE_DEV void argmax_dpp(float& v, int& i) {
    const int vb = __builtin_bit_cast(int, v);
    const float ov = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(vb, vb, CTRL, ROW_MASK, 0xF, false));
    const int oi = __builtin_amdgcn_update_dpp(i, i, CTRL, ROW_MASK, 0xF, false);
    argmax_take(v, i, ov, oi);
}
// Wave-wide argmax, returned wave-uniform: quads, half rows, rows (xor 1, xor 2,
// half-row and row mirrors), then rows 0-1 into row 1 and rows 0-3 into row 3
// (row broadcasts of lanes 15 and 31); lane 63 ends with the whole wave.
MOE_DEV void wave_argmax(float& v, int& i) {
    argmax_dpp<0xB1, 0xF>(v, i);
    argmax_dpp<0x4E, 0xF>(v, i);
    argmax_dpp<0x141, 0xF>(v, i);
    argmax_dpp<0x140, 0xF>(v, i);
    argmax_dpp<0x142, 0xA>(v, i);
    argmax_dpp<0x143, 0xC>(v, i);
    v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), kWave - 1));
    i = __builtin_amdgcn_readlane(i, kWave - 1);
}
MOE_DEV float wave_sum(float x) {
    x += dpp_partner_f<0>(x);
    x += dpp_partner_f<1>(x);
    x += dpp_partner_f<2>(x);
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x142, 0xA, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x143, 0xC, 0xF, false));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), kWave - 1));
}

// Exact selection of one row by a whole wave (the row index is wave-uniform):
// lane l holds experts l + 64*j (j < 4, E <= 256).  K rounds of a wave-wide
// argmax on the fp32 logits, largest first, lower expert index among equal
// values (-0.0 == +0.0); lane r keeps slot r.
MOE_DEV void gate_exact_row(const float* __restrict__ lrow, int t, int E, int K, int lane,
                            int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int* hist) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane + kWave * j;
        v[j] = e < E ? lrow[e] + 0.0f : -INFINITY;
    }
    float mine_v = 0.0f, first_v = 0.0f;
    int mine_i = 0;
    for (int r = 0; r < K; ++r) {
        float bv = v[0];
        int bi = lane;
#pragma unroll
        for (int j = 1; j < 4; ++j) argmax_take(bv, bi, v[j], lane + kWave * j);
        wave_argmax(bv, bi);
        const bool owner = (bi & (kWave - 1)) == lane;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = (owner && j == bi / kWave) ? -INFINITY : v[j];
        mine_v = lane == r ? bv : mine_v;
        mine_i = lane == r ? bi : mine_i;
        if (r == 0) first_v = bv;
    }
    const float ex = lane < K ? expf(mine_v - first_v) : 0.0f;
    const float S = wave_sum(ex);
    if (lane < K) {
        topk_idx[(size_t)t * K + lane] = mine_i;
        topk_w[(size_t)t * K + lane] = ex / S;
        // only non-finite logits (outside the contract) leave mine_i out of range
        if ((unsigned)mine_i < (unsigned)E) atomicAdd(&hist[mine_i], 1);
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
    constexpr int NWAVE = THREADS / kWave;
    constexpr int REG = RPW * EP * 4;              // bytes of one staged pass of a wave
    static_assert(REG % 1024 == 0, "staging region");
    // two regions per wave (the next pass lands while this one is used) when
    // they fit in 128 KB, else one (refilled once this pass's reads are done)
    constexpr int NBUF = NWAVE * 2 * REG <= 128 * 1024 ? 2 : 1;
    constexpr int SPL = (KP + G - 1) / G;          // output slots per lane: r = g + G*i
    __shared__ int hist[256];
    __shared__ __attribute__((aligned(1024))) char stage[VEC ? NWAVE * NBUF * REG : 16];
    __shared__ int flagged[kMaxChunk];  // rows left to the exact path
    __shared__ int n_flagged;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int g = lane % G;
    const int rw = lane / G;
    for (int e = tid; e < E; e += THREADS) hist[e] = 0;
    if (tid == 0) n_flagged = 0;
    __syncthreads();

    const int chunk = blockIdx.x;
    const int t0 = chunk * CH;
    const int t1 = min(T, t0 + CH);

    // Staging copy (E % 4 == 0) of the RPW rows starting at row pb into region
    // `buf` of this wave.  The buffer's range is the chunk, so rows past it read
    // as zeros.
    char* const wstage = stage + wave * NBUF * REG;
    const uint32_t wstage_lds = (uint32_t)(uintptr_t)(lds_void*)wstage;
    const rsrc_t rsrc = make_rsrc(logits + (size_t)t0 * E, (uint32_t)(t1 - t0) * (uint32_t)E * 4u);
    const uint32_t lane_src = 16u * (uint32_t)(lane ^ ((lane >> 3) & 7));
    const int ndma = PAD ? (RPW * E * 4 + 1023) >> 10 : REG / 1024;  // 1 KB copies per pass
    auto stage_rows = [&](int pb, int buf) {
        const uint32_t roff = (uint32_t)(pb - t0) * (uint32_t)E * 4u;
#pragma unroll
        for (int i = 0; i < REG / 1024; ++i)
            if (i < ndma) dma16(rsrc, wstage_lds + buf * REG + i * 1024, roff + i * 1024 + lane_src, 0u);
    };
    // float f of the wave's staged rows in region `buf` (16-byte chunks swizzled)
    auto staged_chunk = [&](int buf, int c) -> const char* {
        return wstage + buf * REG + ((c ^ ((c >> 3) & 7)) << 4);
    };
    if constexpr (VEC) stage_rows(t0 + wave * RPW, 0);

    // Outputs go through buffer stores over the chunk's slice of topk_idx and
    // topk_w; a lane with nothing to store writes past the range, which drops
    // the store.  With staging, a pass's outputs are stored early in the next
    // pass (right after its wait for the staged rows), so that the wait never
    // has to cover stores issued just before it.
    const __amdgpu_buffer_rsrc_t out_idx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(topk_idx + (size_t)t0 * K), (short)0, (t1 - t0) * K * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t out_w = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(topk_w + (size_t)t0 * K), (short)0, (t1 - t0) * K * 4, 0x00020000);
    constexpr uint32_t kDrop = 0x80000000u;  // an offset past any chunk's outputs
    uint32_t pend_off[SPL], pend_idx[SPL], pend_w[SPL];  // outputs not stored yet
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
        pend_off[i] = kDrop;
        pend_idx[i] = 0u;
        pend_w[i] = 0u;
    }
    auto store_pending = [&]() {
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            __builtin_amdgcn_raw_buffer_store_b32(pend_idx[i], out_idx, pend_off[i], 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(pend_w[i], out_w, pend_off[i], 0, 0);
        }
    };

    int pass = 0;
    for (int base = t0 + wave * RPW; base < t1; base += RPB, ++pass) {
        const int t = base + rw;
        const bool valid = t < t1;
        const int buf = NBUF == 2 ? (pass & 1) : 0;
        // ---- keys ----
        // Padding columns get key 0 (below every logit).  Rows past the chunk
        // are computed and discarded: nothing of theirs is stored or counted.
        const float* lrow = logits + (size_t)min(t, T - 1) * E;
        // index bits IMASK - e; V is a power of two, so IMASK - g*V - j == (IMASK - g*V) ^ j
        const uint32_t ibase = IMASK - (uint32_t)(g * V);
        uint32_t key[V];
        if constexpr (VEC) {
            // this pass's rows have landed; with two regions, the next pass's
            // copy goes into the other one, whose reads all completed in the
            // previous pass; then the previous pass's outputs are stored
            __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            if constexpr (NBUF == 2) {
                __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                stage_rows(base + RPB, buf ^ 1);
            }
            store_pending();
            f32x4 x[V / 4];
#pragma unroll
            for (int q = 0; q < V / 4; ++q) {
                const int e0 = g * V + q * 4;
                const int c = (rw * E + (e0 < E ? e0 : 0)) >> 2;  // 16-byte chunk in the region
                x[q] = *reinterpret_cast<const f32x4*>(staged_chunk(buf, c));
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
            // loads are unconditional (column clamped) so that they are all in flight together
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
        uint32_t own[KP];  // the lane's own best KP keys, for the exactness check
#pragma unroll
        for (int i = 0; i < KP; ++i) own[i] = top[i];
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
        // No unchosen key may share the K-th key's prefix.  With several lanes
        // per row: a lane's largest unchosen key is the largest of its own best
        // KP below the K-th key, unless all of those were chosen ("full"); then
        // the lane counts its keys whose prefix reaches the K-th one's, which
        // must be exactly its KP chosen ones.  With one lane per row that count
        // is the whole check (the lane's KP keys are the chosen ones).
        const uint32_t thr = kth & ~IMASK;
        auto count_reaching = [&]() {
            int c = 0;
#pragma unroll
            for (int j = 0; j < V; ++j) c += (key[j] >= thr) ? 1 : 0;
            return c;
        };
        bool exact_fast;
        if constexpr (G == 1) {
            exact_fast = !dup && count_reaching() == K;
        } else {
            uint32_t below = 0u;
#pragma unroll
            for (int i = 0; i < KP; ++i) below = max(below, own[i] < kth ? own[i] : 0u);
            uint32_t extra = 0u;  // a full lane with an unchosen key at the K-th prefix
            if (__builtin_amdgcn_ballot_w64(own[KP - 1] >= kth) != 0)
                extra = (own[KP - 1] >= kth && count_reaching() > KP) ? 1u : 0u;
            below = max(below, dpp_partner<0>(below));
            extra |= dpp_partner<0>(extra);
            if constexpr (G >= 4) { below = max(below, dpp_partner<1>(below)); extra |= dpp_partner<1>(extra); }
            if constexpr (G >= 8) { below = max(below, dpp_partner<2>(below)); extra |= dpp_partner<2>(extra); }
            exact_fast = !dup && extra == 0u && (below >> IB) != (kth >> IB);
        }

        // ---- weights and outputs of accepted rows ----
        // Lane g of the group owns slots r = g + G*i.  Its slot keys are picked
        // from the group-uniform list with a static select chain (no divergent
        // branches), and the exact logits of its slots are read together.
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
        float l0;
        if constexpr (VEC) {
            auto staged = [&](int e) {
                const int f = rw * E + e;  // float index in the region
                return *reinterpret_cast<const float*>(staged_chunk(buf, f >> 2) + ((f & 3) << 2));
            };
            l0 = staged(e0);
#pragma unroll
            for (int i = 0; i < SPL; ++i) xr[i] = staged(er[i]);
            if constexpr (NBUF == 1) {
                // the region is free once these reads are done: refill it
                __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                if (base + RPB < t1) stage_rows(base + RPB, 0);
            }
        } else {
            l0 = lrow[e0];
#pragma unroll
            for (int i = 0; i < SPL; ++i) xr[i] = lrow[er[i]];
        }
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
        const float rS = __builtin_amdgcn_rcpf(S);
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            const int r = g + G * i;
            const bool st = valid && exact_fast && r < K;
            pend_off[i] = st ? (uint32_t)((t - t0) * K + r) * 4u : kDrop;
            pend_idx[i] = (uint32_t)er[i];
            pend_w[i] = __float_as_uint(ex[i] * rS);
            if (st) atomicAdd(&hist[er[i]], 1);
        }
        if constexpr (!VEC) {
            store_pending();
#pragma unroll
            for (int i = 0; i < SPL; ++i) pend_off[i] = kDrop;
        }

        // ---- rows with (near-)ties: listed for the exact path after the loop ----
        const bool flag = valid && !exact_fast && g == 0;
        if (__builtin_amdgcn_ballot_w64(flag) != 0) {
            if (flag) flagged[atomicAdd(&n_flagged, 1)] = t;
        }
    }
    // the last pass's outputs; a copy may still be in flight (the first one of
    // a wave with no rows in this chunk, or with two regions the one past the
    // wave's last pass)
    if constexpr (VEC) {
        store_pending();
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();

    // ---- exact path: one wave per listed row ----
    const int nf = n_flagged;
    for (int i = wave; i < nf; i += NWAVE) {
        const int tf = uniform(flagged[i]);
        gate_exact_row(logits + (size_t)tf * E, tf, E, K, lane, topk_idx, topk_w, hist);
    }
    __syncthreads();
    for (int e = tid; e < E; e += THREADS) blk[(size_t)chunk * E + e] = hist[e];
}

// One workgroup of 1024 threads.  blk is [B, E] (per-chunk counts).  Produces
// counts[e] = sum_b blk[b,e], offsets = exclusive scan of counts with
// offsets[E] = total, and (if blkbase != nullptr) the placement base of every
// chunk: blkbase[b,e] = offsets[e] + sum_{b' < b} blk[b',e].
constexpr int kScanThreads = 1024;
constexpr int kScanBatch = 32;

__global__ __launch_bounds__(kScanThreads) void scan_kernel(const int32_t* __restrict__ blk, int B,
                                                            int E, int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ blkbase,
                                                            int* __restrict__ zero, int nzero) {
    __shared__ int part[kScanThreads];  // [Q][E]: chunk-group sums, then their exclusive prefix
    __shared__ int sc[2][256];          // scan buffers over experts
    const int tid = threadIdx.x;
    for (int i = tid; i < nzero; i += kScanThreads) zero[i] = 0;
    const int Q = kScanThreads / E;  // chunk groups (>= 4 since E <= 256)
    const int e = tid % E;
    const int q = tid / E;
    const bool act = q < Q;
    const int b0 = act ? (int)(((long long)B * q) / Q) : 0;
    const int b1 = act ? (int)(((long long)B * (q + 1)) / Q) : 0;
    if (act) {
        // batches of 32 independent loads (rows clamped into the group's range)
        // keep the latency of the strided reads overlapped
        int s = 0;
        for (int b = b0; b < b1; b += kScanBatch) {
            int x[kScanBatch];
#pragma unroll
            for (int i = 0; i < kScanBatch; ++i) x[i] = blk[(size_t)min(b + i, b1 - 1) * E + e];
#pragma unroll
            for (int i = 0; i < kScanBatch; ++i) s += (b + i < b1) ? x[i] : 0;
        }
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
        for (int b = b0; b < b1; b += kScanBatch) {
            int x[kScanBatch];
#pragma unroll
            for (int i = 0; i < kScanBatch; ++i) x[i] = blk[(size_t)min(b + i, b1 - 1) * E + e];
#pragma unroll
            for (int i = 0; i < kScanBatch; ++i) {
                if (b + i < b1) {
                    blkbase[(size_t)(b + i) * E + e] = run;
                    run += x[i];
                }
            }
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
                       int32_t* blkbase, hipStream_t s, int* zero, int nzero) {
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, blk, B, E, counts, offsets,
                       blkbase, zero, zero != nullptr ? nzero : 0);
    return hipGetLastError();
}

}  // namespace moe
