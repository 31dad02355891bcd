// Router projection, the step upstream of the gate: logits = X Wr (+ bias).
//
// Page [P1] "Optimising MoE with Triton: topk_gating operator fusion in
// practice" section 2.1 starts its fused gating flow from the logit
// computation, and page [P2] "SpMM in MoE: accelerating sparse experts with
// Triton kernels" section 6 computes the gate logits with a linear layer over
// the token's features.  Logits and Wr are fp32; X is the layer's dtype.
//
// bf16 X: a skinny GEMM (N = E <= 256) on bf16 MFMA.  Wr is fp32, so each
// weight is split into two bf16 terms, hi = bf16(w) and lo = bf16(w - hi), and
// both products are accumulated: |w - (hi + lo)| <= 2^-18 |w|, and the
// products of bf16 X with either term are exact in the fp32 accumulator.
// A prep kernel writes hi and lo transposed ([E_pad, d], k-contiguous) into the
// workspace, so that both MFMA operands are 16-byte pieces of k-contiguous rows.
// E <= 64: router_mfma_kernel, each wave one quarter of d, the four sums added
// in wave order; the fused router-gate repeats its arithmetic bit for bit.  For
// E <= 32 both stage their operands through wave-private LDS by DMA in whole
// lines (router_quarter_lds); for 32 < E <= 64 they load them straight into
// registers.  E > 64: the tile kernel (router_tile_kernel) stages 128 tokens
// and 64 experts' hi and lo rows through a shared LDS ring by DMA.
//
// For E a multiple of 128 and few enough tokens (router_gemm_ok), the same
// split runs on the grouped GEMM's SwiGLU kernel instead: hi and lo stay in
// Wr's [d, E] layout as its two weight matrices, every 256 x 128 tile is split
// along K, and a fixup adds the parts and the two terms (launch_router_gemm).
//
// fp32 X, or d not a multiple of 256: one thread per output, fp32 fused
// multiply-adds in index order.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kThreads = 256;

// Wr [d, E] fp32 -> hi, lo [E_pad, d] bf16 (rows e >= E are zero).
__global__ __launch_bounds__(kThreads) void router_split_kernel(const float* __restrict__ Wr, int d, int E,
                                                                int E_pad, uint16_t* __restrict__ hi,
                                                                uint16_t* __restrict__ lo) {
    const size_t n = (size_t)E_pad * d;
    for (size_t q = (size_t)blockIdx.x * kThreads + threadIdx.x; q < n; q += (size_t)gridDim.x * kThreads) {
        const int e = (int)(q / d), i = (int)(q % d);
        const float w = e < E ? Wr[(size_t)i * E + e] : 0.0f;
        const uint16_t h = f32_to_bf16(w);
        hi[q] = h;
        lo[q] = f32_to_bf16(w - bf16_to_f32(h));
    }
}

// Wr [d, E] fp32 -> hi, lo [d, E] bf16 (the same layout), the one-expert
// schedule of the GEMM path (counts = {T}, offsets = {0, T}), and its claim
// counters cleared (nz <= kThreads ints).
__global__ __launch_bounds__(kThreads) void router_split_nc_kernel(const float* __restrict__ Wr, size_t n, int T,
                                                                   uint16_t* __restrict__ hi,
                                                                   uint16_t* __restrict__ lo,
                                                                   int32_t* __restrict__ sched,
                                                                   int* __restrict__ zero, int nz) {
    for (size_t q = (size_t)blockIdx.x * kThreads + threadIdx.x; q < n; q += (size_t)gridDim.x * kThreads) {
        const float w = Wr[q];
        const uint16_t h = f32_to_bf16(w);
        hi[q] = h;
        lo[q] = f32_to_bf16(w - bf16_to_f32(h));
    }
    if (blockIdx.x == 0 && threadIdx.x < 3) sched[threadIdx.x] = threadIdx.x == 1 ? 0 : T;
    if (blockIdx.x == 0 && (int)threadIdx.x < nz) zero[threadIdx.x] = 0;
}

// E <= 32 (one 32-expert block, 32 tokens): the K-quarter loop with its
// operands staged through LDS by DMA, in whole 128-byte lines, instead of
// loaded straight into registers (a fragment load touches 32 rows of 32
// bytes).  Each wave stages its own quarter of d in a region only it uses, so
// no barrier is needed: per 64-k block, 32 X rows and the 8 WP hi and lo rows
// that hold experts (rows past E read as zeros; lanes past 8 WP take zero
// fragments, as rows past E are zero), 128 bytes each, the 16-byte pieces of a
// row XOR-swizzled by row % 8.  NS stages, NS - 1 blocks in flight.  The MFMAs
// run in the register path's order -- k-steps of 16 ascending, the hi term
// before the lo term -- so the sums are the same bits.
template <int WP>
struct RouterQ {
    static constexpr int P = 4 + 2 * WP;                      // 1 KB pieces per stage
    static constexpr int NS = WP == 1 ? 4 : WP == 2 ? 3 : 2;  // stages
    static constexpr int WAVE_BYTES = NS * P * 1024;
    static constexpr size_t LDS = 4 * (size_t)WAVE_BYTES;
};

template <int WP>
MOE_DEV void router_quarter_lds(const uint16_t* __restrict__ X, int T, int t0, int d,
                                const uint16_t* __restrict__ hi, const uint16_t* __restrict__ lo, int E,
                                char* wst, uint32_t wst_lds, int wave, int lane, f32x16& acc) {
    using C = RouterQ<WP>;
    const int l32 = lane & 31, lh = lane >> 5;
    const uint32_t rb = (uint32_t)d * 2u;
    const int ew = min(E, 8 * WP);
    const rsrc_t xs = make_rsrc(X + (size_t)t0 * d, (uint32_t)min(T - t0, 32) * rb);
    const rsrc_t hs = make_rsrc(hi, (uint32_t)ew * rb);
    const rsrc_t ls = make_rsrc(lo, (uint32_t)ew * rb);
    // lane L of a piece writes row 8p + L/8, LDS piece L % 8 = global piece (L % 8) ^ (L / 8)
    const uint32_t lane_off = (uint32_t)(lane >> 3) * rb + (uint32_t)(((lane & 7) ^ (lane >> 3)) << 4);
    const int kq = d / 4, nb = kq / 64;
    const uint32_t k_base = (uint32_t)(wave * kq) * 2u;
    auto issue = [&](int b, int st) __attribute__((always_inline)) {
        const uint32_t ko = k_base + (uint32_t)min(b, nb - 1) * 128u;  // past the end: a harmless reload
        const uint32_t dst = wst_lds + (uint32_t)(st * C::P) * 1024u;
#pragma unroll
        for (int p = 0; p < 4; ++p) dma16(xs, dst + p * 1024, lane_off + 8u * p * rb, ko);
#pragma unroll
        for (int p = 0; p < WP; ++p) dma16(hs, dst + (4 + p) * 1024, lane_off + 8u * p * rb, ko);
#pragma unroll
        for (int p = 0; p < WP; ++p) dma16(ls, dst + (4 + WP + p) * 1024, lane_off + 8u * p * rb, ko);
    };
    const int sw = l32 & 7;
    const bool wrow = l32 < 8 * WP;
    const int wr = (wrow ? l32 : 0) * 128;
#pragma unroll
    for (int b = 0; b < C::NS - 1; ++b) issue(b, b);
    int st = 0;
    for (int b = 0; b < nb; ++b) {
        // block b has landed; the fragments of block b - 1 are all read
        if constexpr (C::NS == 4) __asm__ volatile("s_waitcnt vmcnt(12) lgkmcnt(0)" ::: "memory");
        else if constexpr (C::NS == 3) __asm__ volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");
        else __asm__ volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        issue(b + C::NS - 1, st == 0 ? C::NS - 1 : st - 1);
        const char* sb = wst + st * C::P * 1024;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            const int pc = ((2 * s4 + lh) ^ sw) << 4;
            const bf16x8 xf = *reinterpret_cast<const bf16x8*>(sb + l32 * 128 + pc);
            bf16x8 hf = bf16x8{}, lf = bf16x8{};
            if (wrow) {
                hf = *reinterpret_cast<const bf16x8*>(sb + 4 * 1024 + wr + pc);
                lf = *reinterpret_cast<const bf16x8*>(sb + (4 + WP) * 1024 + wr + pc);
            }
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hf, xf, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf, xf, acc, 0, 0, 0);
        }
        st = st == C::NS - 1 ? 0 : st + 1;
    }
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no DMA outlives the loop
}

// Workgroup tile: 32*TG tokens x 32*NB experts; the four waves split d into
// four quarters and their fp32 sums are added in wave order at the end (fixed
// order: deterministic).  Each weight fragment a wave loads serves its TG
// token groups, which cuts the L2 reads of the split weights by TG.  MFMA operands: a = 32 experts x 16 k of hi or lo,
// b = 16 k x 32 tokens of X, both 8 consecutive k per lane; the accumulator
// holds, in lane l, token l % 32 and experts (i/4)*8 + (l/32)*4 + i%4.
// Workgroups of one XCD (blockIdx mod 8) take the expert groups of the same
// token tile, so that they share its X rows in L2.  WP > 0 (NB = TG = 1): the
// operands go through LDS (router_quarter_lds) in the same MFMA order.
template <int NB, int TG, int WP = 0>
__global__ __launch_bounds__(kThreads) void router_mfma_kernel(const uint16_t* __restrict__ X, int T, int d,
                                                               const uint16_t* __restrict__ hi,
                                                               const uint16_t* __restrict__ lo,
                                                               const float* __restrict__ bias, int E,
                                                               int n_eg, float* __restrict__ logits) {
    constexpr int U = TG > 1 ? 2 : 4;  // k-steps whose operands are loaded together
    __shared__ f32x16 red[4][NB * TG][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int l32 = lane & 31, lh = lane >> 5;
    // block b: XCD b % 8, expert group (b / 8) % n_eg, token tile from the rest
    const int b = blockIdx.x;
    const int eg = (b >> 3) % n_eg;
    const int tt = (b & 7) + 8 * ((b >> 3) / n_eg);
    const int t0 = tt * 32 * TG;
    if (t0 >= T) return;
    const int e0 = eg * 32 * NB;
    const uint16_t* xr[TG];
#pragma unroll
    for (int g = 0; g < TG; ++g)  // rows past T are computed and discarded
        xr[g] = X + (size_t)min(t0 + g * 32 + l32, T - 1) * d + lh * 8;
    const size_t woff = (size_t)(e0 + l32) * d + lh * 8;
    const int kq = d / 4;  // this wave's quarter of d
    const int kb = wave * kq;

    f32x16 acc[TG][NB];
#pragma unroll
    for (int g = 0; g < TG; ++g)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[g][j][i] = 0.0f;

    if constexpr (WP > 0) {
        static_assert(NB == 1 && TG == 1, "LDS staging: one 32-expert block of 32 tokens");
        extern __shared__ __attribute__((aligned(1024))) char rq_stage[];
        char* wst = rq_stage + wave * RouterQ<WP>::WAVE_BYTES;
        router_quarter_lds<WP>(X, T, t0, d, hi, lo, E, wst, (uint32_t)(uintptr_t)(lds_void*)wst, wave, lane,
                               acc[0][0]);
    } else {
        for (int k0 = kb; k0 < kb + kq; k0 += 16 * U) {
            bf16x8 xf[U][TG], hf[U][NB], lf[U][NB];
    #pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = k0 + u * 16;
    #pragma unroll
                for (int g = 0; g < TG; ++g) xf[u][g] = *reinterpret_cast<const bf16x8*>(xr[g] + k);
    #pragma unroll
                for (int j = 0; j < NB; ++j) {
                    // One expert block (E <= 32): the padding rows past E are zeros, so
                    // their lanes load nothing; with E = 8 that is 3/4 of the weight reads.
                    if (NB > 1 || e0 + j * 32 + l32 < E) {
                        hf[u][j] = *reinterpret_cast<const bf16x8*>(hi + woff + (size_t)j * 32 * d + k);
                        lf[u][j] = *reinterpret_cast<const bf16x8*>(lo + woff + (size_t)j * 32 * d + k);
                    } else {
                        hf[u][j] = bf16x8{};
                        lf[u][j] = bf16x8{};
                    }
                }
            }
    #pragma unroll
            for (int u = 0; u < U; ++u)
    #pragma unroll
                for (int g = 0; g < TG; ++g)
    #pragma unroll
                    for (int j = 0; j < NB; ++j) {
                        acc[g][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hf[u][j], xf[u][g], acc[g][j], 0, 0, 0);
                        acc[g][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf[u][j], xf[u][g], acc[g][j], 0, 0, 0);
                    }
        }
    }
#pragma unroll
    for (int g = 0; g < TG; ++g)
#pragma unroll
        for (int j = 0; j < NB; ++j) red[wave][g * NB + j][lane] = acc[g][j];
    __syncthreads();
    // the NB*TG (token group, expert block) pieces are finished by the waves in turn
    for (int pc = wave; pc < NB * TG; pc += 4) {
        const int g = pc / NB, j = pc % NB;
        f32x16 s = red[0][pc][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) s += red[w][pc][lane];
        const int t = t0 + g * 32 + l32;
        if (t < T) {
            float* orow = logits + (size_t)t * E;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int e = e0 + j * 32 + (i >> 2) * 8 + lh * 4 + (i & 3);
                if (e < E) orow[e] = s[i] + (bias != nullptr ? bias[e] : 0.0f);
            }
        }
    }
}

// Router tile kernel for E > 64 (bf16 X, d % 64 == 0).  Workgroup tile: 128
// tokens x 64 experts, both terms of the split.  K goes in blocks of 64 through
// a 4-stage LDS ring filled by DMA.  A 32 KB stage holds 128 X rows and 128
// weight rows (the tile's 64 hi rows, then its 64 lo rows) of 128 bytes each;
// the 16-byte pieces of row r are XOR-swizzled by r % 8, so the fragment reads
// are free of bank conflicts.  A DMA instruction reads 8 whole 128-byte lines,
// where loading MFMA fragments straight from global memory touches 32 lines
// for the same 1 KB.  Wave w takes tokens 64 (w / 2) .. +63 (two groups of 32)
// and experts 32 (w % 2) .. +31; every accumulator takes its k-steps of 16 in
// ascending order, the hi term before the lo term.
constexpr int kRtTok = 128, kRtExp = 64, kRtStage = 32768, kRtStages = 4;
constexpr size_t kRtLds = (size_t)kRtStages * kRtStage;

__global__ __launch_bounds__(kThreads, 1) void router_tile_kernel(const uint16_t* __restrict__ X, int T, int d,
                                                                  const uint16_t* __restrict__ hi,
                                                                  const uint16_t* __restrict__ lo,
                                                                  const float* __restrict__ bias, int E, int n_eg,
                                                                  float* __restrict__ logits) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = uniform(tid / kWave);
    const int l32 = lane & 31, lh = lane >> 5;
    // block b: XCD b % 8, expert group (b / 8) % n_eg, token tile from the rest
    const int b = blockIdx.x;
    const int eg = (b >> 3) % n_eg;
    const int tt = (b & 7) + 8 * ((b >> 3) / n_eg);
    const int t0 = tt * kRtTok;
    if (t0 >= T) return;
    const int e0 = eg * kRtExp;
    const int nK = d / 64;
    const uint32_t row_bytes = (uint32_t)d * 2u;
    const uint32_t lds_base = uniform((int)(uint32_t)(uintptr_t)(lds_void*)smem);

    // DMA: waves 0-1 fill the X half of a stage (pieces 0-15), wave 2 the hi
    // rows (pieces 16-23), wave 3 the lo rows (pieces 24-31).  Piece q holds
    // region rows 8q' .. 8q'+7 (q' = q within the wave's matrix); lane L writes
    // row 8q' + L/8 at LDS piece L % 8, which holds the row's global piece
    // (L % 8) ^ (L / 8).  X rows past T read as zeros (buffer range).
    const bool xw = wave < 2;
    const int tv = min(T - t0, kRtTok);
    const rsrc_t rs = xw ? make_rsrc(X + (size_t)t0 * d, (uint32_t)tv * row_bytes)
                         : make_rsrc((wave == 2 ? hi : lo) + (size_t)e0 * d, (uint32_t)kRtExp * row_bytes);
    const int q0 = xw ? wave * 8 : 0;  // first piece of the wave within its matrix
    uint32_t voff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        voff[i] = (uint32_t)(8 * (q0 + i) + (lane >> 3)) * row_bytes + (uint32_t)(((lane & 7) ^ (lane >> 3)) << 4);
    const uint32_t dst0 = lds_base + (uint32_t)(wave * 8) * 1024u;
    auto issue = [&](int kb, int st) __attribute__((always_inline)) {
        const uint32_t ko = (uint32_t)min(kb, nK - 1) * 128u;  // past the end: a harmless reload
        const uint32_t dst = dst0 + (uint32_t)st * kRtStage;
#pragma unroll
        for (int i = 0; i < 8; ++i) dma16(rs, dst + i * 1024, voff[i], ko);
    };

    // Fragments: lane l supplies row l % 32 at k = 8 (l / 32) .. +7 of a 16-k
    // step, that is piece 2s + l / 32 of the row for step s of a block.
    const int wt = wave >> 1, we = wave & 1;
    const int sw = l32 & 7;  // every fragment row here is l32 plus a multiple of 8
    const int x_rd = (wt * 64 + l32) * 128;
    const int h_rd = 16384 + (we * 32 + l32) * 128;
    const int l_rd = 16384 + (64 + we * 32 + l32) * 128;

    f32x16 acc[2];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[g][i] = 0.0f;

    issue(0, 0);
    issue(1, 1);
    issue(2, 2);
    for (int kb = 0; kb < nK; ++kb) {
        const int st = kb & (kRtStages - 1);
        // this wave's pieces of block kb have landed (two blocks stay in flight);
        // the barrier makes every wave's pieces visible and retires the reads of
        // block kb - 1, whose stage the refill below overwrites
        __asm__ volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        issue(kb + 3, (kb + 3) & (kRtStages - 1));
        const char* sb = smem + st * kRtStage;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            const int pc = ((2 * s4 + lh) ^ sw) << 4;
            const bf16x8 x0 = *reinterpret_cast<const bf16x8*>(sb + x_rd + pc);
            const bf16x8 x1 = *reinterpret_cast<const bf16x8*>(sb + x_rd + 32 * 128 + pc);
            const bf16x8 hf = *reinterpret_cast<const bf16x8*>(sb + h_rd + pc);
            const bf16x8 lf = *reinterpret_cast<const bf16x8*>(sb + l_rd + pc);
            acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hf, x0, acc[0], 0, 0, 0);
            acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf, x0, acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hf, x1, acc[1], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf, x1, acc[1], 0, 0, 0);
        }
    }
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no DMA outlives the workgroup

    // lane l holds token l % 32 of its group and experts (i/4)*8 + (l/32)*4 + i%4
    // of its 32-expert block in acc[g][i]
    const bool vec = (E & 3) == 0;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const int t = t0 + wt * 64 + g * 32 + l32;
        if (t >= T) continue;
        float* orow = logits + (size_t)t * E;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = e0 + we * 32 + q * 8 + lh * 4;
            f32x4 v = {acc[g][4 * q], acc[g][4 * q + 1], acc[g][4 * q + 2], acc[g][4 * q + 3]};
            if (vec && e + 3 < E) {
                if (bias != nullptr) v += *reinterpret_cast<const f32x4*>(bias + e);
                *reinterpret_cast<f32x4*>(orow + e) = v;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (e + j < E) orow[e + j] = v[j] + (bias != nullptr ? bias[e + j] : 0.0f);
            }
        }
    }
}

// The router projection fused with the gate (page [P1] section 2.1: logit
// computation, softmax and top-k in one pass; page [P4] section 1: the K best
// of E scores per token), for E <= 64.  A workgroup computes the logits of one
// tile of 32 tokens exactly as router_mfma_kernel does (the same MFMA order
// over k within each wave's quarter of d, the four waves' sums added in wave
// order, then the bias), so they equal moe_router's logits bit for bit; they
// never leave the workgroup unless `logits` asks for them.  From LDS, LPT
// lanes per token (8 experts each) then take K rounds of a group argmax: the
// largest logit, the lower expert index among equal ones (-0.0 == +0.0), best
// first.  Weights exp(l_k - l_0) / sum_j exp(l_j - l_0), the sum in rank
// order.  The tile's expert counts go to blk[tile, E] (integer LDS atomics).
template <int NB, int WP = 0>
__global__ __launch_bounds__(kThreads) void router_gate_kernel(
    const uint16_t* __restrict__ X, int T, int d, const uint16_t* __restrict__ hi, const uint16_t* __restrict__ lo,
    const float* __restrict__ bias, int E, int K, float* __restrict__ logits, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ blk) {
    constexpr int U = 4;
    constexpr int EP = 32 * NB;   // padded expert count
    constexpr int LPT = EP / 8;   // gate lanes per token
    constexpr int TT = kRouterGateTokens;
    static_assert(TT == 32, "one 32-row MFMA token group per tile");
    __shared__ f32x16 red[4][NB][kWave];
    __shared__ float lgs[TT][EP + 1];
    __shared__ int hist[EP];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int l32 = lane & 31, lh = lane >> 5;
    const int tile = blockIdx.x;
    const int t0 = tile * TT;
    if (t0 >= T) return;
    if (tid < EP) hist[tid] = 0;
    // rows past T are computed and discarded
    const uint16_t* xr = X + (size_t)min(t0 + l32, T - 1) * d + lh * 8;
    const size_t woff = (size_t)l32 * d + lh * 8;
    const int kq = d / 4;
    const int kb = wave * kq;

    f32x16 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][i] = 0.0f;
    if constexpr (WP > 0) {
        static_assert(NB == 1, "LDS staging: one 32-expert block");
        extern __shared__ __attribute__((aligned(1024))) char rq_stage[];
        char* wst = rq_stage + wave * RouterQ<WP>::WAVE_BYTES;
        router_quarter_lds<WP>(X, T, t0, d, hi, lo, E, wst, (uint32_t)(uintptr_t)(lds_void*)wst, wave, lane,
                               acc[0]);
    } else {
        for (int k0 = kb; k0 < kb + kq; k0 += 16 * U) {
            bf16x8 xf[U], hf[U][NB], lf[U][NB];
    #pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = k0 + u * 16;
                xf[u] = *reinterpret_cast<const bf16x8*>(xr + k);
    #pragma unroll
                for (int j = 0; j < NB; ++j) {
                    if (NB > 1 || l32 < E) {
                        hf[u][j] = *reinterpret_cast<const bf16x8*>(hi + woff + (size_t)j * 32 * d + k);
                        lf[u][j] = *reinterpret_cast<const bf16x8*>(lo + woff + (size_t)j * 32 * d + k);
                    } else {
                        hf[u][j] = bf16x8{};
                        lf[u][j] = bf16x8{};
                    }
                }
            }
    #pragma unroll
            for (int u = 0; u < U; ++u)
    #pragma unroll
                for (int j = 0; j < NB; ++j) {
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hf[u][j], xf[u], acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf[u][j], xf[u], acc[j], 0, 0, 0);
                }
        }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) red[wave][j][lane] = acc[j];
    __syncthreads();
    if (wave < NB) {  // wave j finishes expert block j
        const int j = wave;
        f32x16 sm = red[0][j][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) sm += red[w][j][lane];
        const int t = t0 + l32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int e = j * 32 + (i >> 2) * 8 + lh * 4 + (i & 3);
            const float v = e < E ? sm[i] + (bias != nullptr ? bias[e] : 0.0f) : 0.0f;
            lgs[l32][e] = v;
            if (logits != nullptr && t < T && e < E) logits[(size_t)t * E + e] = v;
        }
    }
    __syncthreads();

    if (tid < TT * LPT) {  // whole waves: LPT * 32 is 128 or 256 lanes
        const int tk = tid / LPT, g = tid % LPT;
        const int t = t0 + tk;
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = lgs[tk][g * 8 + j];
        constexpr int kNone = 0x7fffffff;
        unsigned taken = 0u;
        float sv[8];
        int si[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            sv[r] = 0.0f;
            si[r] = 0;
            if (r < K) {
                float bv = 0.0f;
                int bi = kNone;
#pragma unroll
                for (int j = 0; j < 8; ++j) {  // ascending index: strict > keeps the lower one
                    const int e = g * 8 + j;
                    const bool ok = e < E && !((taken >> j) & 1u);
                    if (ok && (bi == kNone || v[j] > bv)) {
                        bv = v[j];
                        bi = e;
                    }
                }
#pragma unroll
                for (int o = 1; o < LPT; o <<= 1) {
                    const float ov = __shfl_xor(bv, o, kWave);
                    const int oi = __shfl_xor(bi, o, kWave);
                    if (oi != kNone && (bi == kNone || ov > bv || (ov == bv && oi < bi))) {
                        bv = ov;
                        bi = oi;
                    }
                }
                sv[r] = bv;
                si[r] = bi;
                if (bi >= g * 8 && bi < g * 8 + 8) taken |= 1u << (bi - g * 8);
            }
        }
        float ex[8];
        float S = 0.0f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            ex[r] = r < K ? expf(sv[r] - sv[0]) : 0.0f;
            S += ex[r];
        }
        const float rS = __builtin_amdgcn_rcpf(S);
        if (t < T) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                if (r < K && r % LPT == g) {
                    topk_idx[(size_t)t * K + r] = si[r];
                    topk_w[(size_t)t * K + r] = ex[r] * rS;
                    atomicAdd(&hist[si[r]], 1);
                }
            }
        }
    }
    __syncthreads();
    if (tid < E) blk[(size_t)tile * E + tid] = hist[tid];
}

// One thread per (token, expert), fp32 FMAs over d in index order.
MOE_DEV float load_x(const float* p) { return *p; }
MOE_DEV float load_x(const uint16_t* p) { return bf16_to_f32(*p); }
template <typename XT>
__global__ __launch_bounds__(kThreads) void router_fma_kernel(const XT* __restrict__ X, int T, int d,
                                                              const float* __restrict__ Wr,
                                                              const float* __restrict__ bias, int E,
                                                              float* __restrict__ logits) {
    const size_t q = (size_t)blockIdx.x * kThreads + threadIdx.x;
    if (q >= (size_t)T * E) return;
    const int t = (int)(q / E), e = (int)(q % E);
    const XT* xr = X + (size_t)t * d;
    float s = 0.0f;
    for (int i = 0; i < d; ++i) s = fmaf(load_x(xr + i), Wr[(size_t)i * E + e], s);
    logits[q] = s + (bias != nullptr ? bias[e] : 0.0f);
}

int router_nb(int E) { return E <= 32 ? 1 : 2; }
int router_tg(int E) { return E <= 32 ? 1 : 4; }  // token groups of 32 per workgroup

// The MFMA kernel's four waves take d/4 each, 64 at a time.
bool router_mfma_ok(int dtype, int d) { return dtype == 1 && d % 256 == 0; }

}  // namespace

// The GEMM path's layout: hi, lo [d, E]; 256 bytes for its schedule; the
// GEMM's split slots.  It is reserved whenever the shapes allow the path (it
// also depends on T), and it is never smaller than the transposed layout.
static bool router_gemm_shape(int dtype, int d, int E) { return router_mfma_ok(dtype, d) && router_gemm_ok(1, d, E); }
static size_t router_hilo_bytes(int d, int E) { return ((2 * (size_t)d * E * sizeof(uint16_t)) + 255) / 256 * 256; }

size_t router_split_bytes(int dtype, int d, int E) {
    if (!router_mfma_ok(dtype, d)) return 0;
    const int eb = 32 * router_nb(E);
    const size_t e_pad = (size_t)((E + eb - 1) / eb) * eb;
    const size_t transposed = 2 * e_pad * (size_t)d * sizeof(uint16_t);
    if (!router_gemm_shape(dtype, d, E)) return transposed;
    return std::max(transposed, router_hilo_bytes(d, E) + 256 + ffn_split_bytes(1, d, E));
}

// Weight pieces of 8 rows staged per block by the E <= 32 kernels (0: the
// register path, for 32 < E <= 64).
static int router_wp(int E) { return E <= 8 ? 1 : E <= 16 ? 2 : E <= 32 ? 4 : 0; }

template <int WP>
static hipError_t launch_router_q(const uint16_t* X, int T, int d, const uint16_t* hi, const uint16_t* lo,
                                  const float* bias, int E, float* logits, dim3 grid, hipStream_t s) {
    const hipError_t aerr = hipFuncSetAttribute((const void*)router_mfma_kernel<1, 1, WP>,
                                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)RouterQ<WP>::LDS);
    if (aerr != hipSuccess) return aerr;
    hipLaunchKernelGGL((router_mfma_kernel<1, 1, WP>), grid, dim3(kThreads), RouterQ<WP>::LDS, s, X, T, d, hi, lo,
                       bias, E, 1, logits);
    return hipGetLastError();
}

template <int WP>
static hipError_t launch_router_gate_q(const uint16_t* X, int T, int d, const uint16_t* hi, const uint16_t* lo,
                                       const float* bias, int E, int K, float* logits, int32_t* idx, float* w,
                                       int32_t* blk, dim3 grid, hipStream_t s) {
    const hipError_t aerr = hipFuncSetAttribute((const void*)router_gate_kernel<1, WP>,
                                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)RouterQ<WP>::LDS);
    if (aerr != hipSuccess) return aerr;
    hipLaunchKernelGGL((router_gate_kernel<1, WP>), grid, dim3(kThreads), RouterQ<WP>::LDS, s, X, T, d, hi, lo,
                       bias, E, K, logits, idx, w, blk);
    return hipGetLastError();
}

bool router_gate_ok(int dtype, int d, int E) { return router_mfma_ok(dtype, d) && E <= 64; }

hipError_t launch_router_gate(const void* X, int T, int d, int E, int K, const float* Wr, const float* bias,
                              float* logits, int32_t* idx, float* w, int32_t* blk, void* split, hipStream_t s) {
    if (!router_gate_ok(1, d, E) || K < 1 || K > 8 || K > E) return hipErrorInvalidValue;
    const int nb = router_nb(E);
    const int e_pad = 32 * nb;
    uint16_t* hi = static_cast<uint16_t*>(split);
    uint16_t* lo = hi + (size_t)e_pad * d;
    const size_t n = (size_t)e_pad * d;
    const unsigned sgrid = (unsigned)std::min<size_t>((n + kThreads - 1) / kThreads, 4096);
    hipLaunchKernelGGL(router_split_kernel, dim3(sgrid), dim3(kThreads), 0, s, Wr, d, E, e_pad, hi, lo);
    const dim3 grid((unsigned)((T + kRouterGateTokens - 1) / kRouterGateTokens));
    const uint16_t* Xb = static_cast<const uint16_t*>(X);
    switch (router_wp(E)) {
        case 1: return launch_router_gate_q<1>(Xb, T, d, hi, lo, bias, E, K, logits, idx, w, blk, grid, s);
        case 2: return launch_router_gate_q<2>(Xb, T, d, hi, lo, bias, E, K, logits, idx, w, blk, grid, s);
        case 4: return launch_router_gate_q<4>(Xb, T, d, hi, lo, bias, E, K, logits, idx, w, blk, grid, s);
        default: break;
    }
    // 32 < E <= 64: two expert blocks, operands loaded straight into registers
    hipLaunchKernelGGL(router_gate_kernel<2>, grid, dim3(kThreads), 0, s, Xb, T, d, hi, lo, bias, E, K, logits, idx,
                       w, blk);
    return hipGetLastError();
}

hipError_t launch_router(const void* X, int dtype, int T, int d, int E, const float* Wr, const float* bias,
                         float* logits, void* split, hipStream_t s) {
    if (!router_mfma_ok(dtype, d)) {
        const size_t n = (size_t)T * E;
        const dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
        if (dtype == 1)
            hipLaunchKernelGGL(router_fma_kernel<uint16_t>, grid, dim3(kThreads), 0, s,
                               static_cast<const uint16_t*>(X), T, d, Wr, bias, E, logits);
        else
            hipLaunchKernelGGL(router_fma_kernel<float>, grid, dim3(kThreads), 0, s, static_cast<const float*>(X),
                               T, d, Wr, bias, E, logits);
        return hipGetLastError();
    }
    if (router_gemm_ok(T, d, E)) {
        uint16_t* hi = static_cast<uint16_t*>(split);
        uint16_t* lo = hi + (size_t)d * E;
        int32_t* sched = reinterpret_cast<int32_t*>(static_cast<char*>(split) + router_hilo_bytes(d, E));
        float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(sched) + 256);
        const size_t n = (size_t)d * E;
        const unsigned sgrid = (unsigned)std::min<size_t>((n + kThreads - 1) / kThreads, 4096);
        const int nz = ffn_ticket_ints();
        if (nz > kThreads) return hipErrorInvalidValue;
        hipLaunchKernelGGL(router_split_nc_kernel, dim3(sgrid), dim3(kThreads), 0, s, Wr, n, T, hi, lo, sched,
                           ffn_tickets(part), nz);
        return launch_router_gemm(static_cast<const uint16_t*>(X), hi, lo, T, d, E, sched, sched + 1, bias, logits,
                                  part, true, s);
    }
    const int nb = router_nb(E);
    const int eb = 32 * nb;
    const int n_eg = (E + eb - 1) / eb;
    const int e_pad = n_eg * eb;
    uint16_t* hi = static_cast<uint16_t*>(split);
    uint16_t* lo = hi + (size_t)e_pad * d;
    const size_t n = (size_t)e_pad * d;
    const unsigned sgrid = (unsigned)std::min<size_t>((n + kThreads - 1) / kThreads, 4096);
    hipLaunchKernelGGL(router_split_kernel, dim3(sgrid), dim3(kThreads), 0, s, Wr, d, E, e_pad, hi, lo);
    if (E > 64) {
        const hipError_t aerr = hipFuncSetAttribute((const void*)router_tile_kernel,
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)kRtLds);
        if (aerr != hipSuccess) return aerr;
        // token tiles rounded up to a multiple of 8 (one per XCD); blocks past T exit at once
        const int tiles = (((T + kRtTok - 1) / kRtTok) + 7) / 8 * 8;
        hipLaunchKernelGGL(router_tile_kernel, dim3((unsigned)(tiles * n_eg)), dim3(kThreads), kRtLds, s,
                           static_cast<const uint16_t*>(X), T, d, hi, lo, bias, E, n_eg, logits);
        return hipGetLastError();
    }
    // token tiles rounded up to a multiple of 8 (one per XCD); blocks past T exit at once
    const int tt = 32 * router_tg(E);
    const int tiles = (((T + tt - 1) / tt) + 7) / 8 * 8;
    const dim3 grid((unsigned)(tiles * n_eg));
    const uint16_t* Xb = static_cast<const uint16_t*>(X);
    switch (router_wp(E)) {
        case 1: return launch_router_q<1>(Xb, T, d, hi, lo, bias, E, logits, grid, s);
        case 2: return launch_router_q<2>(Xb, T, d, hi, lo, bias, E, logits, grid, s);
        case 4: return launch_router_q<4>(Xb, T, d, hi, lo, bias, E, logits, grid, s);
        default: break;
    }
    // 32 < E <= 64: two expert blocks, operands loaded straight into registers
    hipLaunchKernelGGL((router_mfma_kernel<2, 4>), grid, dim3(kThreads), 0, s, Xb, T, d, hi, lo, bias, E, n_eg,
                       logits);
    return hipGetLastError();
}

}  // namespace moe
