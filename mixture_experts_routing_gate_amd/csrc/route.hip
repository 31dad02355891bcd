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

constexpr int kGateThreads = 256;
constexpr int kPerLane = 8;  // logits held by each lane of a row group

// One workgroup per chunk of `CH` tokens; rows are spread over groups of G
// lanes (64/G rows per wave per pass).  Selection is exact on fp32 logits:
// K rounds of a group-wide argmax, largest value first and the lower expert
// index among equal values (floating-point equality, so -0.0 == +0.0 after
// the canonicalising +0.0f).  Weights are exp(l_k - l_0) / sum_j exp(l_j - l_0),
// which equals the softmax renormalised over the K winners.
template <int G>
__global__ __launch_bounds__(kGateThreads) void gate_kernel(const float* __restrict__ logits, int T,
                                                            int E, int K, int CH,
                                                            int32_t* __restrict__ topk_idx,
                                                            float* __restrict__ topk_w,
                                                            int32_t* __restrict__ blk) {
    constexpr int RPW = kWave / G;  // rows per wave per pass
    constexpr int RPB = RPW * (kGateThreads / kWave);
    __shared__ int hist[256];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int g = lane % G;
    const int rw = lane / G;
    for (int e = tid; e < E; e += kGateThreads) hist[e] = 0;
    __syncthreads();

    const int chunk = blockIdx.x;
    const int t0 = chunk * CH;
    const int t1 = min(T, t0 + CH);
    const bool vec4 = (E & 3) == 0;

    for (int base = t0 + wave * RPW; base < t1; base += RPB) {
        const int t = base + rw;
        const bool valid = t < t1;
        float v[kPerLane];
        const float* row = logits + (size_t)t * E;
        if (vec4) {
#pragma unroll
            for (int q = 0; q < kPerLane / 4; ++q) {
                const int e0 = g * kPerLane + q * 4;
                f32x4 x = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
                if (valid && e0 < E) x = *reinterpret_cast<const f32x4*>(row + e0);
                v[q * 4 + 0] = x[0];
                v[q * 4 + 1] = x[1];
                v[q * 4 + 2] = x[2];
                v[q * 4 + 3] = x[3];
            }
        } else {
#pragma unroll
            for (int j = 0; j < kPerLane; ++j) {
                const int e = g * kPerLane + j;
                v[j] = (valid && e < E) ? row[e] : -INFINITY;
            }
        }
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) v[j] = v[j] + 0.0f;  // -0.0 -> +0.0

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
                for (int j = 1; j < kPerLane; ++j)
                    if (v[j] > bv) {
                        bv = v[j];
                        bj = j;
                    }
                const float M = group_max<G>(bv);
                const int cand = (bv == M) ? g * kPerLane + bj : 0x7fffffff;
                const int I = group_min<G>(cand);
#pragma unroll
                for (int j = 0; j < kPerLane; ++j)
                    if (g * kPerLane + j == I) v[j] = -INFINITY;
                sv[r] = M;
                si[r] = I;
            }
        }

        // Lane g of the group owns slots r = g, g+G, ...: one exp per owned slot.
        float ex[8];
        float part = 0.0f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            ex[r] = 0.0f;
            if (r < K && (r % G) == g) {
                ex[r] = expf(sv[r] - sv[0]);
                part += ex[r];
            }
        }
        const float S = group_sum<G>(part);
        if (valid) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                if (r < K && (r % G) == g) {
                    topk_idx[(size_t)t * K + r] = si[r];
                    topk_w[(size_t)t * K + r] = ex[r] / S;
                    // only non-finite logits (outside the contract) can leave si out of range
                    if ((unsigned)si[r] < (unsigned)E) atomicAdd(&hist[si[r]], 1);
                }
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kGateThreads) blk[(size_t)chunk * E + e] = hist[e];
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
        int s = 0;
        for (int b = b0; b < b1; ++b) s += blk[(size_t)b * E + e];
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
        for (int b = b0; b < b1; ++b) {
            blkbase[(size_t)b * E + e] = run;
            run += blk[(size_t)b * E + e];
        }
    }
}

template <int G>
hipError_t launch_gate_g(const float* logits, int T, int E, int K, int32_t* idx, float* w,
                         int32_t* blk, hipStream_t s) {
    const int CH = chunk_tokens(T);
    const int B = num_chunks(T);
    hipLaunchKernelGGL(gate_kernel<G>, dim3(B), dim3(kGateThreads), 0, s, logits, T, E, K, CH, idx, w,
                       blk);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gate(const float* logits, int T, int E, int K, int32_t* idx, float* w,
                       int32_t* blk, hipStream_t s) {
    if (E <= 8) return launch_gate_g<1>(logits, T, E, K, idx, w, blk, s);
    if (E <= 16) return launch_gate_g<2>(logits, T, E, K, idx, w, blk, s);
    if (E <= 32) return launch_gate_g<4>(logits, T, E, K, idx, w, blk, s);
    if (E <= 64) return launch_gate_g<8>(logits, T, E, K, idx, w, blk, s);
    if (E <= 128) return launch_gate_g<16>(logits, T, E, K, idx, w, blk, s);
    return launch_gate_g<32>(logits, T, E, K, idx, w, blk, s);
}

hipError_t launch_scan(const int32_t* blk, int B, int E, int32_t* counts, int32_t* offsets,
                       int32_t* blkbase, hipStream_t s) {
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, blk, B, E, counts, offsets,
                       blkbase);
    return hipGetLastError();
}

}  // namespace moe
