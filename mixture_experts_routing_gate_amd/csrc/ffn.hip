// Step 4 of the MoE layer forward: the grouped expert MLP.
//
// Page [P4] "MoE architecture optimisation and SonicMoE practice" section 1
// (each expert is a two-layer MLP, first layer through SiLU) and section 2.2
// (the SwiGLU activation fused into the GEMM epilogue); page [P3] "Triton
// optimisation speeds up matrix computation for Mixture-of-Experts models"
// (all experts' GEMMs in one launch; a persistent grid sized to the machine
// that walks a tile list).  The tile list is derived on the device from the
// per-expert counts: expert e owns ceil(count_e / BM) row tiles times N/BN
// column tiles, so empty experts cost nothing and no host sync is needed.
//
//   FFN1: Act[r] = SiLU(Xp[r] W1[e]) * (Xp[r] W3[e])   (both products in one tile)
//   FFN2: Y[r]   = Act[r] W2[e]
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kThreads = 256;

// Builds s_start[0..E] = exclusive prefix over experts of (row tiles * NT) in
// LDS.  Must be called by all threads of the block.
template <int BM>
__device__ void build_schedule(const int32_t* __restrict__ counts, int E, int NT, int rows,
                               int* s_start, int* s_tmp) {
    const int tid = threadIdx.x;
    int v = 0;
    if (tid < E) v = ((min(max(counts[tid], 0), rows) + BM - 1) / BM) * NT;
    s_tmp[tid] = v;
    __syncthreads();
    for (int sh = 1; sh < 256; sh <<= 1) {  // inclusive scan over 256 slots
        const int x = (tid >= sh) ? s_tmp[tid - sh] : 0;
        __syncthreads();
        s_tmp[tid] += x;
        __syncthreads();
    }
    if (tid < E) s_start[tid + 1] = s_tmp[tid];
    if (tid == 0) s_start[0] = 0;
    __syncthreads();
}

// Expert owning global tile `tile`: the last e with s_start[e] <= tile.
__device__ __forceinline__ int find_expert(const int* s_start, int E, int tile) {
    int lo = 0, hi = E;  // answer in [lo, hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_start[mid] <= tile) lo = mid; else hi = mid;
    }
    return lo;
}

// SiLU(h1) * h3 with SiLU(z) = z / (1 + e^-z) (page [P4] section 2.2).  The
// quotient uses the hardware reciprocal (1 ulp) rather than an IEEE division
// sequence: the result is rounded to bf16 right after, and the division was
// most of the SwiGLU epilogue's cost.  Large negative z gives e^-z = inf and a
// zero reciprocal, so the limit 0 comes out as it should.
MOE_DEV float silu_mul(float h1, float h3) { return h1 * __builtin_amdgcn_rcpf(1.0f + __expf(-h1)) * h3; }

// bf16 MFMA tile kernel.  Block tile 128 x 128 x 64, four waves in 2 x 2, each
// wave 64 x 64 as 2 x 2 v_mfma_f32_32x32x16_bf16 tiles (x2 for the W1/W3 pair).
// A [rows, Kd] is K-contiguous; B [Kd, N] is N-contiguous and is transposed
// into LDS so that both MFMA operands read 8 consecutive k per lane.
template <bool DUAL>
__global__ __launch_bounds__(kThreads, 2) void ffn_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1,
    uint16_t* __restrict__ C, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    int E, int Kd, int N, int rows) {
    constexpr int BM = 128, BN = 128, BK = 64, LDK = BK + 8;
    constexpr int NB = DUAL ? 2 : 1;
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[NB][BN * LDK];
    __shared__ int s_start[257];
    __shared__ int s_tmp[256];

    const int NT = N / BN;
    build_schedule<BM>(counts, E, NT, rows, s_start, s_tmp);
    const int total = s_start[E];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, lh = lane >> 5;

    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const int e = find_expert(s_start, E, tile);
        const int cnt = min(max(counts[e], 0), rows);
        const int mt = (cnt + BM - 1) / BM;
        const int local = tile - s_start[e];
        const int m_tile = local % mt;
        const int n_tile = local / mt;
        const int r0 = offsets[e] + m_tile * BM;
        // rows of this tile that exist; never past the end of A/C whatever counts/offsets hold
        const int rows_valid = (r0 < 0 || r0 >= rows) ? 0 : min(min(BM, cnt - m_tile * BM), rows - r0);
        const size_t row0 = (size_t)max(r0, 0);
        const int n0 = n_tile * BN;
        const uint16_t* Bp[2] = {B0 + (size_t)e * Kd * N, DUAL ? B1 + (size_t)e * Kd * N : nullptr};

        f32x16 acc[NB][2][2];
        #pragma unroll
        for (int m = 0; m < NB; ++m)
            #pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                #pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    #pragma unroll
                    for (int i = 0; i < 16; ++i) acc[m][mi][ni][i] = 0.0f;

        for (int k0 = 0; k0 < Kd; k0 += BK) {
            __syncthreads();
            #pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = tid + kThreads * i;
                const int r = c >> 3;
                const int kc = (c & 7) << 3;
                u32x4 val = {0u, 0u, 0u, 0u};
                if (r < rows_valid) val = *reinterpret_cast<const u32x4*>(A + (row0 + r) * Kd + k0 + kc);
                *reinterpret_cast<u32x4*>(As + r * LDK + kc) = val;
            }
            #pragma unroll
            for (int m = 0; m < NB; ++m) {
                #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = tid + kThreads * i;
                    const int kr = c >> 4;
                    const int nc = (c & 15) << 3;
                    const u32x4 val =
                        *reinterpret_cast<const u32x4*>(Bp[m] + (size_t)(k0 + kr) * N + n0 + nc);
                    #pragma unroll
                    for (int j = 0; j < 8; ++j)
                        Bs[m][(nc + j) * LDK + kr] = (uint16_t)(val[j >> 1] >> (16 * (j & 1)));
                }
            }
            __syncthreads();
            #pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
                bf16x8 a[2], b[NB][2];
                #pragma unroll
                for (int mi = 0; mi < 2; ++mi)
                    a[mi] = *reinterpret_cast<const bf16x8*>(As + (wm * 64 + mi * 32 + l32) * LDK + ks * 16 + lh * 8);
                #pragma unroll
                for (int m = 0; m < NB; ++m)
                    #pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
                        b[m][ni] = *reinterpret_cast<const bf16x8*>(Bs[m] + (wn * 64 + ni * 32 + l32) * LDK + ks * 16 + lh * 8);
                #pragma unroll
                for (int m = 0; m < NB; ++m)
                    #pragma unroll
                    for (int mi = 0; mi < 2; ++mi)
                        #pragma unroll
                        for (int ni = 0; ni < 2; ++ni)
                            acc[m][mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[m][ni], acc[m][mi][ni], 0, 0, 0);
            }
        }
        // 32x32 accumulator layout: element i of lane l is row (i/4)*8 + (l/32)*4 + i%4, column l%32.
        #pragma unroll
        for (int mi = 0; mi < 2; ++mi)
            #pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                #pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = wm * 64 + mi * 32 + (i >> 2) * 8 + lh * 4 + (i & 3);
                    const int col = n0 + wn * 64 + ni * 32 + l32;
                    if (row < rows_valid) {
                        float v = acc[0][mi][ni][i];
                        if (DUAL) v = silu_mul(v, acc[NB - 1][mi][ni][i]);
                        C[(row0 + row) * N + col] = f32_to_bf16(v);
                    }
                }
    }
}

constexpr int kBM256 = 256;  // rows per tile of the pipelined kernel

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: in each 16-lane group, lane i receives element i%4 of the
// 8-byte chunks addressed by lanes i/4, 4+i/4, 8+i/4 and 12+i/4 -- a 4 x 16 ->
// 16 x 4 transpose of 16-bit values, which is the MFMA operand layout for an
// N-contiguous B tile.
MOE_DEV bf16x4 lds_read_tr(const char* l) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(l));
    return __builtin_bit_cast(bf16x4, v);
}

// v_mfma_f32_16x16x32_bf16 with the accumulator held in AGPRs and tied to the
// result.  Written as inline assembly because with the builtin the register
// allocator leaves dst and srcC apart in a loop of 64 accumulators and then
// shuffles them through copies at every step.  The compiler does not see these
// as MFMAs, so the waits it would insert around them are made by hand: the
// first K-step uses the zero-accumulator form (no VALU write of the
// accumulators precedes an MFMA that reads them), the loaded operands reach
// the MFMAs straight from LDS reads (waited for by the compiler, which tracks
// the asm operands), and mfma16_drain separates the last MFMA from any read of
// its results by more wait states than the MFMA's passes.
MOE_DEV void mfma16(f32x4& acc, const bf16x8& a, const bf16x8& b) {
    __asm__ volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
MOE_DEV void mfma16_first(f32x4& acc, const bf16x8& a, const bf16x8& b) {
    __asm__ volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
}
MOE_DEV void mfma16_drain(f32x4 (&acc)[8][8]) {
    __asm__ volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]), "+a"(acc[0][4]),
                       "+a"(acc[0][5]), "+a"(acc[0][6]), "+a"(acc[0][7]), "+a"(acc[1][0]), "+a"(acc[1][1]),
                       "+a"(acc[1][2]), "+a"(acc[1][3]), "+a"(acc[1][4]), "+a"(acc[1][5]), "+a"(acc[1][6]),
                       "+a"(acc[1][7]));
    #pragma unroll
    for (int mi = 2; mi < 8; mi += 2)
        __asm__ volatile(""
                         : "+a"(acc[mi][0]), "+a"(acc[mi][1]), "+a"(acc[mi][2]), "+a"(acc[mi][3]), "+a"(acc[mi][4]),
                           "+a"(acc[mi][5]), "+a"(acc[mi][6]), "+a"(acc[mi][7]), "+a"(acc[mi + 1][0]),
                           "+a"(acc[mi + 1][1]), "+a"(acc[mi + 1][2]), "+a"(acc[mi + 1][3]), "+a"(acc[mi + 1][4]),
                           "+a"(acc[mi + 1][5]), "+a"(acc[mi + 1][6]), "+a"(acc[mi + 1][7]));
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel with a 5-stage LDS pipeline (used when d % 256 == 0 and
// n % 128 == 0).  Tiles of 256 x 256 per CU, 4 waves of 128 x 128, K advancing
// 32 at a time through five 32 KB LDS stages (all 160 KB of a CU's LDS; the
// tile schedule lives in registers):
//  * DMA is buffer_load ... lds: one scalar buffer resource per matrix, a
//    fixed 32-bit per-lane offset per tile and a scalar offset per K-step, so
//    issuing a load costs no vector ALU work.
//  * One barrier per K-step, at its start: it publishes step kt+1's stage
//    (every wave first waits for its own part of that DMA) and retires the
//    stage of step kt-1 (every read of it completed before the barrier), which
//    is then refilled with step kt+4 -- three K-steps of lead time.
//  * The K-loop has no branches: near the end of K the refill index is clamped
//    to the last step (a duplicate load into a stage nobody reads again), so
//    the schedule below can be pinned with scheduling fences.  The 8 DMAs of a
//    step go out one per MFMA right after the barrier; the fragment reads of
//    the next sub-step run under the current sub-step's 16 MFMAs.
//  * Each 32-row B stage is stored as two 128-column halves so that every DMA
//    instruction reads a single matrix (W1 or W3 for the SwiGLU GEMM).
// ---------------------------------------------------------------------------
constexpr int kP4BK = 32, kP4Stage = 32768, kP4Stages = 5, kP4Lds = kP4Stages * kP4Stage;
// LDS word that passes a claimed work ticket to all waves (in the last stage).
constexpr int kP4TicketOff = (kP4Stages - 1) * kP4Stage;
// Claim counters of the dynamic schedule: one per XCD, 64 bytes apart.
constexpr int kTicketInts = 8 * 16;

// The tile schedule of the pipelined kernel, held in registers (E <= 256): lane
// l holds experts 4l..4l+3, and expert e owns the tiles [start_e, start_e +
// ceil(count_e / 256) * NT) in expert order.  Returns the expert owning `tile`
// (-1 if none) and writes its first tile to *start and the number of tiles to
// *total.  All lanes of the wave must call it.
MOE_DEV int sched_lookup(const int32_t* __restrict__ counts, int E, int NT, int rows, int lane, int tile,
                         int* start, int* total) {
    int v[4];
    #pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane * 4 + j;
        const int c = e < E ? min(max(counts[e], 0), rows) : 0;
        v[j] = ((c + kBM256 - 1) / kBM256) * NT;
    }
    const int p0 = v[0], p1 = p0 + v[1], p2 = p1 + v[2], p3 = p2 + v[3];
    int x = p3;  // inclusive scan of the per-lane totals
    #pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
    const int base = x - p3;
    *total = __shfl(x, kWave - 1, kWave);
    const int b0 = base, b1 = base + p0, b2 = base + p1, b3 = base + p2, b4 = base + p3;
    int hit = -1, st = 0;
    if (tile >= b0 && tile < b1) { hit = 0; st = b0; }
    if (tile >= b1 && tile < b2) { hit = 1; st = b1; }
    if (tile >= b2 && tile < b3) { hit = 2; st = b2; }
    if (tile >= b3 && tile < b4) { hit = 3; st = b3; }
    const unsigned long long m = __ballot(hit >= 0);
    if (m == 0ull) return -1;
    const int src = __builtin_ctzll(m);
    *start = __shfl(st, src, kWave);
    return src * 4 + __shfl(hit, src, kWave);
}

// Number of tiles of the pipelined kernel's schedule with at most 128 rows
// (the short-tile layouts).  All lanes of the wave must call it.
MOE_DEV int count_short_tiles(const int32_t* __restrict__ counts, int E, int NT, int rows, int lane) {
    int n = 0;
    #pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane * 4 + j;
        const int c = e < E ? min(max(counts[e], 0), rows) : 0;
        const int rem = c % kBM256;
        n += (rem > 0 && rem <= 128) ? NT : 0;
    }
    #pragma unroll
    for (int o = 1; o < kWave; o <<= 1) n += __shfl_xor(n, o, kWave);
    return uniform(n);
}

// Rows and columns of pipelined-kernel tile `tile` (wave-uniform results).
struct TileGeom {
    int e, r0, rows_valid, n0;
};
MOE_DEV bool tile_geom(const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets, int E, int NT,
                       int OUTW, int rows, int lane, int tile, TileGeom& t) {
    int first = 0, total = 0;
    const int e = uniform(sched_lookup(counts, E, NT, rows, lane, tile, &first, &total));
    if (e < 0) return false;
    const int cnt = min(max(counts[e], 0), rows);
    const int mt = (cnt + kBM256 - 1) / kBM256;
    const int local = tile - uniform(first);
    const int m_tile = local % mt;
    const int n_tile = local / mt;
    t.e = e;
    t.r0 = offsets[e] + m_tile * kBM256;
    t.rows_valid = (t.r0 < 0 || t.r0 >= rows) ? 0 : min(min(kBM256, cnt - m_tile * kBM256), rows - t.r0);
    t.n0 = n_tile * OUTW;
    return true;
}

// The same schedule held in registers for the whole launch (counts and
// offsets do not change during it): lane l keeps experts 4l..4l+3's clamped
// row counts and offsets and the first tile of expert 4l, so that a tile's
// geometry costs a few cross-lane operations instead of two rounds of global
// loads.  (The other tile-range boundaries are re-derived from the counts
// when a tile is decoded: nine long-lived registers instead of thirteen keep
// the SwiGLU epilogue from spilling them.)
struct SchedRegs {
    int b0;      // first tile of expert 4l
    int cnt[4];  // row counts of experts 4l..4l+3, clamped into [0, rows]
    int off[4];  // their offsets
    int total;   // tiles of the whole schedule
};
MOE_DEV SchedRegs sched_regs(const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets, int E,
                             int NT, int rows, int lane) {
    SchedRegs sr;
    int v[4];
    #pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane * 4 + j;
        sr.cnt[j] = e < E ? min(max(counts[e], 0), rows) : 0;
        sr.off[j] = e < E ? offsets[e] : 0;
        v[j] = ((sr.cnt[j] + kBM256 - 1) / kBM256) * NT;
    }
    const int p3 = v[0] + v[1] + v[2] + v[3];
    int x = p3;  // inclusive scan of the per-lane totals
    #pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
    sr.b0 = x - p3;
    sr.total = uniform(__shfl(x, kWave - 1, kWave));
    return sr;
}
// tile_geom on the register schedule (wave-uniform results; all lanes call it).
MOE_DEV bool tile_geom_regs(const SchedRegs& sr, int NT, int OUTW, int rows, int lane, int tile, TileGeom& t) {
    int hit = -1, st = 0, c = 0, o = 0;
    int lo = sr.b0;  // first tile of expert 4l+j
    #pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int hi = lo + ((sr.cnt[j] + kBM256 - 1) / kBM256) * NT;
        if (tile >= lo && tile < hi) {
            hit = j;
            st = lo;
            c = sr.cnt[j];
            o = sr.off[j];
        }
        lo = hi;
    }
    const unsigned long long m = __ballot(hit >= 0);
    if (m == 0ull) return false;
    const int src = __builtin_ctzll(m);
    const int e = src * 4 + uniform(__shfl(hit, src, kWave));
    const int first = uniform(__shfl(st, src, kWave));
    const int cnt = uniform(__shfl(c, src, kWave));
    const int off = uniform(__shfl(o, src, kWave));
    const int mt = (cnt + kBM256 - 1) / kBM256;
    const int local = tile - first;
    const int m_tile = local % mt;
    const int n_tile = local / mt;
    t.e = e;
    t.r0 = off + m_tile * kBM256;
    t.rows_valid = (t.r0 < 0 || t.r0 >= rows) ? 0 : min(min(kBM256, cnt - m_tile * kBM256), rows - t.r0);
    t.n0 = n_tile * OUTW;
    return true;
}

// Split of the last, partial round of tiles over the idle workgroups: with
// G workgroups and `total` tiles, the first R*G tiles are computed whole and
// each of the Tr = total - R*G remaining ones in S parts of consecutive K-steps
// (S = min(G / Tr, KT / 4), parts of whole groups of 4 K-steps).  Part p (of
// Tr*S) writes its fp32 accumulators to slot p of the split workspace; the
// fixup kernel adds a tile's S slots in order and runs the epilogue.
struct SplitPlan {
    int R, Tr, S;
};
MOE_DEV SplitPlan split_plan(int total, int G, int KT, bool enabled) {
    SplitPlan sp;
    sp.R = total / G;
    sp.Tr = total - sp.R * G;
    sp.S = (enabled && sp.Tr > 0) ? min(G / sp.Tr, KT / 4) : 1;
    return sp;
}
constexpr int kPartFloats = 256 * 256;  // one 256 x 256 fp32 tile per slot

// Output of one 32-row slice sl of a wave's 128 x 128 quadrant (row blocks
// 2sl, 2sl+1 of 16) from the 16x16x32 accumulators a[mm][ni]: lane l holds row
// l%16 of block mm and output columns ni*16 + 4*(l/16) .. +3; bf16, rows past
// rows_valid skipped.  With DUAL, a[mm][ni] (ni < 4) is the W1 part and
// a[mm][ni + 4] the W3 part of the same columns, giving SiLU(W1 part) * (W3 part).
// (The lane index is re-derived here rather than kept live from the kernel's
// start: after the K-loop registers are scarce, and a spilled lane index would
// cost a scratch reload per tile.)
template <bool DUAL>
MOE_DEV void store_rows(const f32x4 (&a)[2][8], int sl, uint16_t* __restrict__ C, int r0, int rows_valid, int n0,
                        int N, int wm, int wn) {
    int lane = __lane_id();
    __asm__ volatile("" : "+v"(lane));  // keeps the row math here instead of hoisted (and spilled)
    const int s16 = lane & 15, g16 = lane >> 4;
    #pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
        const int m = wm * 128 + sl * 32 + mm * 16 + s16;
        if (m < rows_valid) {
            uint16_t* crow = C + (size_t)(r0 + m) * N + n0 + (DUAL ? wn * 64 : wn * 128) + 4 * g16;
            #pragma unroll
            for (int ni = 0; ni < (DUAL ? 4 : 8); ++ni) {
                float v[4];
                #pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[j] = a[mm][ni][j];
                    if (DUAL) v[j] = silu_mul(v[j], a[mm][ni + 4][j]);
                }
                uint2 pk;
                pk.x = pack_bf16x2(v[0], v[1]);
                pk.y = pack_bf16x2(v[2], v[3]);
                *reinterpret_cast<uint2*>(crow + ni * 16) = pk;
            }
        }
    }
}

// The same output through LDS, for whole tiles: the slice (32 rows of the
// wave's 128 x 128 quadrant) is written to the wave's own 8 KB of stage 0 --
// the parts of it that only this wave's DMAs fill, so no other wave's reads
// or loads touch them -- and read back as 16-byte pieces of whole row
// segments, so that each store instruction writes 4 rows of 256 bytes (8 rows
// of 128 bytes for the SwiGLU GEMM) instead of 64 pieces of 8 bytes.  Staged
// rows are XOR-swizzled by 16-byte piece so that writes and reads are free of
// bank conflicts.  Every wave must be done reading the stages, and this wave's
// own loads into them must be complete.
// Staged row r: SwiGLU rows at wave*4K + r*128; otherwise rows 0..15 at
// wave*4K + r*256 and rows 16..31 at 16K + wave*4K + (r-16)*256.
template <bool DUAL>
MOE_DEV char* staged_row(char* smem, int wave, int r) {
    return DUAL ? smem + wave * 4096 + r * 128 : smem + (r >> 4) * 16384 + wave * 4096 + (r & 15) * 256;
}
template <bool DUAL>
MOE_DEV int staged_swz(int r, int c) { return DUAL ? (c ^ ((r >> 1) & 7)) : (c ^ (r & 15)); }

// Writes slice sl of the accumulators to the staging rows, rounded to bf16 (with
// DUAL, SiLU(W1 part) * (W3 part) first).  Lane l writes row (l%16) of each
// block, 8 bytes per column block: staged columns ni*16 + 4*(l/16) .. +3.
// An accumulator element read out of its AGPR at this point of the program
// (the register allocator otherwise copies whole accumulator blocks to VGPRs
// early, which raises the epilogue's register peak until long-lived values
// spill).  After the K-loop's drain, so no MFMA hazard is pending.
MOE_DEV float acc_read(float a) {
    float v;
    __asm__ volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}

template <bool DUAL>
MOE_DEV void stage_slice(const f32x4 (&acc)[8][8], int sl, char* smem, int wave, int s16, int g16) {
    #pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
        const int r = mm * 16 + s16;
        char* wr = staged_row<DUAL>(smem, wave, r);
        #pragma unroll
        for (int ni = 0; ni < (DUAL ? 4 : 8); ++ni) {
            float v[4];
            #pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[j] = acc_read(acc[2 * sl + mm][ni][j]);
                if (DUAL) v[j] = silu_mul(v[j], acc_read(acc[2 * sl + mm][ni + 4][j]));
            }
            uint2 pk;
            pk.x = pack_bf16x2(v[0], v[1]);
            pk.y = pack_bf16x2(v[2], v[3]);
            const int c = ni * 2 + (g16 >> 1);  // 16-byte piece of the staged row
            *reinterpret_cast<uint2*>(wr + staged_swz<DUAL>(r, c) * 16 + (g16 & 1) * 8) = pk;
            // (keeps the accumulator reads of the next pieces from being hoisted here,
            // which would raise the register peak of the epilogue)
            if constexpr (DUAL) __builtin_amdgcn_sched_barrier(0);
        }
    }
}

template <bool DUAL>
MOE_DEV void store_rows_lds(const f32x4 (&acc)[8][8], int sl, char* smem, uint16_t* __restrict__ C, int r0,
                            int rows_valid, int n0, int N, int wave, int wm, int wn) {
    int lane = __lane_id();
    __asm__ volatile("" : "+v"(lane));
    constexpr int CH = DUAL ? 8 : 16;   // 16-byte pieces per staged row (64 or 128 columns)
    constexpr int RPI = kWave / CH;     // rows per store instruction
    stage_slice<DUAL>(acc, sl, smem, wave, lane & 15, lane >> 4);
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int c = lane % CH;
    const int colb = n0 + (DUAL ? wn * 64 : wn * 128) + c * 8;
    u32x4 val[32 / RPI];
    #pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
        const int r = i * RPI + lane / CH;
        val[i] = *reinterpret_cast<const u32x4*>(staged_row<DUAL>(smem, wave, r) + staged_swz<DUAL>(r, c) * 16);
    }
    #pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
        const int r = i * RPI + lane / CH;
        const int m = wm * 128 + sl * 32 + r;
        if (m < rows_valid) *reinterpret_cast<u32x4*>(C + (size_t)(r0 + m) * N + colb) = val[i];
    }
}

// The SwiGLU GEMM's pre-activations as they are (for the backward, which needs
// H1 = Xp W1 and H3 = Xp W3 themselves): slice sl of the W1 part to C and of
// the W3 part to C + h3_off, bf16.  The slice is staged as the plain GEMM's is
// (128 staged columns per wave: 0..63 the W1 part, 64..127 the W3 part of the
// wave's 64 output columns) and read back as 16-byte pieces of row segments.
MOE_DEV void store_rows_lds_raw(const f32x4 (&acc)[8][8], int sl, char* smem, uint16_t* __restrict__ C,
                                size_t h3_off, int r0, int rows_valid, int n0, int N, int wave, int wm, int wn) {
    int lane = __lane_id();
    __asm__ volatile("" : "+v"(lane));
    constexpr int CH = 16, RPI = kWave / CH;
    stage_slice<false>(acc, sl, smem, wave, lane & 15, lane >> 4);
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int c = lane % CH;
    uint16_t* const dst = (c < 8 ? C : C + h3_off) + n0 + wn * 64 + (c & 7) * 8;
    u32x4 val[32 / RPI];
    #pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
        const int r = i * RPI + lane / CH;
        val[i] = *reinterpret_cast<const u32x4*>(staged_row<false>(smem, wave, r) + staged_swz<false>(r, c) * 16);
    }
    #pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
        const int r = i * RPI + lane / CH;
        const int m = wm * 128 + sl * 32 + r;
        if (m < rows_valid) *reinterpret_cast<u32x4*>(dst + (size_t)(r0 + m) * N) = val[i];
    }
}

// Output of row slice mi of a short tile (rows mi*32 .. mi*32+31, all four
// waves): wave w holds output columns w*32.. (SwiGLU: a[0] the W1 part, a[1]
// the W3 part) or w*64 + ni*32.. (plain GEMM).
template <bool DUAL>
MOE_DEV void store_rows_short(const f32x16 (&a)[2], int mi, uint16_t* __restrict__ C, int r0, int rows_valid,
                              int n0, int N, int wave) {
    int lane = __lane_id();
    __asm__ volatile("" : "+v"(lane));
    const int l32 = lane & 31, lh = lane >> 5;
    const int m = mi * 32 + l32;
    if (m < rows_valid) {
        uint16_t* crow = C + (size_t)(r0 + m) * N;
        #pragma unroll
        for (int ni = 0; ni < (DUAL ? 1 : 2); ++ni) {
            #pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v[4];
                #pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[j] = a[ni][q * 4 + j];
                    if (DUAL) v[j] = silu_mul(v[j], a[1][q * 4 + j]);
                }
                const int col = n0 + (DUAL ? wave * 32 : wave * 64 + ni * 32) + q * 8 + lh * 4;
                uint2 pk;
                pk.x = pack_bf16x2(v[0], v[1]);
                pk.y = pack_bf16x2(v[2], v[3]);
                *reinterpret_cast<uint2*>(crow + col) = pk;
            }
        }
    }
}

// store_rows_short<true>'s layout without the product: the W1 part (a[0]) to
// C and the W3 part (a[1]) to C + h3_off.
MOE_DEV void store_rows_short_raw(const f32x16 (&a)[2], int mi, uint16_t* __restrict__ C, size_t h3_off, int r0,
                                  int rows_valid, int n0, int N, int wave) {
    int lane = __lane_id();
    __asm__ volatile("" : "+v"(lane));
    const int l32 = lane & 31, lh = lane >> 5;
    const int m = mi * 32 + l32;
    if (m < rows_valid) {
        #pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint16_t* crow = C + (h ? h3_off : 0) + (size_t)(r0 + m) * N;
            #pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = n0 + wave * 32 + q * 8 + lh * 4;
                uint2 pk;
                pk.x = pack_bf16x2(a[h][q * 4], a[h][q * 4 + 1]);
                pk.y = pack_bf16x2(a[h][q * 4 + 2], a[h][q * 4 + 3]);
                *reinterpret_cast<uint2*>(crow + col) = pk;
            }
        }
    }
}

// The SwiGLU backward fused into the epilogue of dA = dY W2^T (page [P4]
// section 2.2: dH and dS formed in the epilogue of the GEMM that produces dA,
// so that dA never travels through memory).  For each element of a tile,
// with h1, h3 the stored pre-activations of the same row and column and w the
// row's routing weight: sig = 1 / (1 + e^-h1), s = h1 sig,
//   dh1 = w dA h3 sig (1 + h1 (1 - sig)),  dh3 = w dA s,  aw = w s h3,
// and dS of the row = sum over all n columns of dA s h3, gathered as one fp32
// partial per 64 columns (ds_part[row, col / 64], in column order inside the
// 64) and added in column-block order by a later kernel.  dA is rounded to
// bf16 first, as when it is stored.
struct BwdEpi {
    const uint16_t* H1;    // [rows, n]
    const uint16_t* H3;    // [rows, n]
    uint16_t* dH;          // [rows, 2n]: dh1 | dh3
    uint16_t* aw;          // [rows, n] or null
    const float* wrow;     // [rows]: routing weight of each expert-sorted row
    float* ds_part;        // [rows, n / 64]
};

// 8 consecutive columns (one 16-byte piece) of a row: dA bits in `ga`, h1 and
// h3 bits in a1, a3.  Returns the dS contribution summed in column order.
MOE_DEV float swiglu_bwd_piece(const u32x4& ga, const u32x4& a1, const u32x4& a3, float w, u32x4& o1, u32x4& o3,
                               u32x4& oa) {
    float ds = 0.0f;
    #pragma unroll
    for (int i = 0; i < 4; ++i) {
        float r1[2], r3[2], ra[2];
        #pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const float h1 = bf16_to_f32((uint16_t)(a1[i] >> (16 * hh)));
            const float h3 = bf16_to_f32((uint16_t)(a3[i] >> (16 * hh)));
            const float g = bf16_to_f32((uint16_t)(ga[i] >> (16 * hh)));
            // the hardware reciprocal and exponential, as in the forward's SiLU
            // (the results are rounded to bf16 right after)
            const float sig = __builtin_amdgcn_rcpf(1.0f + __expf(-h1));
            const float s1 = h1 * sig;
            ds = fmaf(g, s1 * h3, ds);
            const float wg = w * g;
            r1[hh] = wg * h3 * sig * (1.0f + h1 * (1.0f - sig));
            r3[hh] = wg * s1;
            ra[hh] = w * (s1 * h3);
        }
        o1[i] = pack_bf16x2(r1[0], r1[1]);
        o3[i] = pack_bf16x2(r3[0], r3[1]);
        oa[i] = pack_bf16x2(ra[0], ra[1]);
    }
    return ds;
}

// store_rows_lds<false>'s staging, then the SwiGLU backward on each staged
// 16-byte piece instead of a store of dA, for the four 32-row slices of the
// wave's quadrant.  The H1, H3 pieces and row weights of slice mi + 1 are
// requested before slice mi is computed, so that their latency overlaps it.
// Lanes 16q..16q+15 hold one row's 128 columns (8 per lane); each half of them
// (64 columns) adds its dS parts with three butterfly steps, and the first
// lane of the half writes the slot.
MOE_DEV void bwd_rows_lds(const f32x4 (&acc)[8][8], char* smem, int r0, int rows_valid, int n0, int N, int wave,
                          int wm, int wn, const BwdEpi& ep) {
    int lane = __lane_id();
    __asm__ volatile("" : "+v"(lane));
    constexpr int CH = 16, RPI = kWave / CH, NI = 32 / RPI;
    auto row_at = [&](int r) -> char* { return staged_row<false>(smem, wave, r); };
    auto swz = [](int r, int c) { return staged_swz<false>(r, c); };
    const int c = lane % CH;
    const int col = n0 + wn * 128 + c * 8;
    const int nslots = N / 64;
    const int slot = (n0 + wn * 128) / 64 + (c >> 3);
    u32x4 a1[2][NI], a3[2][NI];
    float w[2][NI];
    auto fetch = [&](int mi, int buf) {
        #pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int m = wm * 128 + mi * 32 + i * RPI + lane / CH;
            const size_t row = (size_t)(r0 + min(m, rows_valid - 1));  // clamped: rows past the tile are not stored
            a1[buf][i] = *reinterpret_cast<const u32x4*>(ep.H1 + row * N + col);
            a3[buf][i] = *reinterpret_cast<const u32x4*>(ep.H3 + row * N + col);
            w[buf][i] = ep.wrow[row];
        }
    };
    fetch(0, 0);
    #pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int buf = mi & 1;
        if (mi + 1 < 4) fetch(mi + 1, buf ^ 1);
        stage_slice<false>(acc, mi, smem, wave, lane & 15, lane >> 4);
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        u32x4 ga[NI];
        #pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int r = i * RPI + lane / CH;
            ga[i] = *reinterpret_cast<const u32x4*>(row_at(r) + swz(r, c) * 16);
        }
        #pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int m = wm * 128 + mi * 32 + i * RPI + lane / CH;
            const size_t row = (size_t)(r0 + m);
            u32x4 o1, o3, oa;
            float ds = swiglu_bwd_piece(ga[i], a1[buf][i], a3[buf][i], w[buf][i], o1, o3, oa);
            ds += __shfl_xor(ds, 1, kWave);
            ds += __shfl_xor(ds, 2, kWave);
            ds += __shfl_xor(ds, 4, kWave);
            if (m < rows_valid) {
                *reinterpret_cast<u32x4*>(ep.dH + row * 2 * N + col) = o1;
                *reinterpret_cast<u32x4*>(ep.dH + row * 2 * N + N + col) = o3;
                if (ep.aw != nullptr) *reinterpret_cast<u32x4*>(ep.aw + row * N + col) = oa;
                if ((c & 7) == 0) ep.ds_part[row * nslots + slot] = ds;
            }
        }
    }
}

// The same for a short tile (store_rows_short<false>'s layout): lane l holds
// row mi*32 + l%32 and, in 4-column pieces, half of this wave's 64 columns;
// the two lanes of a row add their dS parts.
MOE_DEV void bwd_rows_short(const f32x16 (&a)[2], int mi, int r0, int rows_valid, int n0, int N, int wave,
                            const BwdEpi& ep) {
    int lane = __lane_id();
    __asm__ volatile("" : "+v"(lane));
    const int l32 = lane & 31, lh = lane >> 5;
    const int m = mi * 32 + l32;
    const size_t row = (size_t)(r0 + min(m, rows_valid - 1));
    const float w = ep.wrow[row];
    float ds = 0.0f;
    #pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        #pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int col = n0 + wave * 64 + ni * 32 + q * 8 + lh * 4;
            const uint2 h1 = *reinterpret_cast<const uint2*>(ep.H1 + row * N + col);
            const uint2 h3 = *reinterpret_cast<const uint2*>(ep.H3 + row * N + col);
            u32x4 ga, a1, a3, o1, o3, oa;
            ga[0] = pack_bf16x2(a[ni][q * 4], a[ni][q * 4 + 1]);
            ga[1] = pack_bf16x2(a[ni][q * 4 + 2], a[ni][q * 4 + 3]);
            ga[2] = 0u;
            ga[3] = 0u;
            a1 = u32x4{h1.x, h1.y, 0u, 0u};
            a3 = u32x4{h3.x, h3.y, 0u, 0u};
            ds += swiglu_bwd_piece(ga, a1, a3, w, o1, o3, oa);
            if (m < rows_valid) {
                *reinterpret_cast<uint2*>(ep.dH + row * 2 * N + col) = uint2{o1[0], o1[1]};
                *reinterpret_cast<uint2*>(ep.dH + row * 2 * N + N + col) = uint2{o3[0], o3[1]};
                if (ep.aw != nullptr) *reinterpret_cast<uint2*>(ep.aw + row * N + col) = uint2{oa[0], oa[1]};
            }
        }
    }
    ds += __shfl_xor(ds, 32, kWave);
    if (m < rows_valid && lh == 0) ep.ds_part[row * (N / 64) + (n0 + wave * 64) / 64] = ds;
}

// Slot layout: per wave the 8 x 8 accumulator blocks of 4 floats per lane, as
// float4 vectors [wave][row block][column block][lane], so that each store and
// load is 1 KB per wave.
MOE_DEV size_t part_index(int wave, int mi, int ni, int lane) {
    return ((size_t)((wave * 8 + mi) * 8 + ni) * kWave + lane);
}

// BT (plain GEMM only): B is given k-contiguous, as the transpose of each
// expert's [N, kb] row-major matrix -- B0 for K-steps below kb / 32 and, when
// Kd = 2 kb, B1 for the rest (C = A [B0^T ; B1^T]).  Its tile is staged like
// A's (256 rows of the N side, 64 bytes of K each) and its fragments are read
// like A's, so the backward multiplies by W2^T and [W1^T ; W3^T] without
// transposing the weights first.
template <bool DUAL, bool BT = false, bool BWD = false>
__global__ __launch_bounds__(kThreads, 1) void ffn_p4_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1,
    uint16_t* __restrict__ C, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    int E, int Kd, int N, int rows, float* __restrict__ part, int* __restrict__ ticket_ctr,
    const int32_t* __restrict__ gather, int gK, int xrows, int kb, BwdEpi bwd) {
    static_assert(!(DUAL && BT), "the k-contiguous B is for the plain GEMM");
    // BWD selects the epilogue the backward needs: for the plain GEMM (dA) the
    // fused SwiGLU backward, for the SwiGLU GEMM the pre-activations H1, H3
    // stored as they are (H3 at C + rows * N).
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    constexpr int OUTW = DUAL ? 128 : 256;
    const int NT = N / OUTW;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = uniform(tid / kWave);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, lh = lane >> 5;
    const int g16 = lane >> 4, s16 = lane & 15;
    const SchedRegs sreg = sched_regs(counts, offsets, E, NT, rows, lane);
    const int total = sreg.total;
    // Claim tiles from the counters only when at least one tile in eight is
    // short.  With tiles of equal length the fixed order keeps the 32
    // workgroups of an XCD in step along K, so that they share the K-slices
    // of their panels in L2; claiming staggers them and costs a few percent.
    int* const tickets = (ticket_ctr != nullptr && 8 * count_short_tiles(counts, E, NT, rows, lane) > total)
                             ? ticket_ctr : nullptr;

    // LDS fragment addresses (byte offsets into a stage).  Whole tiles run on
    // v_mfma_f32_16x16x32_bf16, where lane l supplies row (or output column)
    // l%16 of a 16-wide block at k = 8*(l/16) .. 8*(l/16)+7 of the step's 32.
    // Under the card's power cap this form sustains a higher clock than
    // 32x32x16 for the same work (measured with both on register data:
    // 2.02 against 1.77 GHz at 96% MFMA busy).  Short tiles use 32x32x16.
    // A row r, k-chunk c of 8 elements sits at r*64 + ((c ^ ((r/4)%4)) * 16);
    // fragment mi (rows wm*128 + mi*16 ..) at a16_rd + mi*1024.
    const int a16_rd = (wm * 128 + s16) * 64 + ((g16 ^ ((s16 >> 2) & 3)) << 4);
    // B k-row k, column n of half h sits at 16K + h*8K + k*256 + (n%8)*2 +
    // ((n/8) ^ 4*(k%4) ^ 2*((k/8)%2)) * 16.  The transposing read gives lane l
    // column l%16 of a 16-column block at four consecutive k-rows: lane c of a
    // 16-lane group addresses k-row c/4 and columns 4*(c%4) .. +3.  The XOR
    // terms keep the 16-byte pieces that one read instruction touches in
    // distinct banks.
    const int b_x = (s16 >> 2) << 2;
    const int b16_lane = 16384 + (g16 * 8 + (s16 >> 2)) * 256 + (s16 & 1) * 8;
    int b16_rd[8];
    #pragma unroll
    for (int ni = 0; ni < 8; ++ni) {
        const int half = DUAL ? (ni >> 2) : wn;
        const int nn = DUAL ? (wn * 64 + (ni & 3) * 16) : ni * 16;
        b16_rd[ni] = b16_lane + half * 8192 + ((((nn >> 3) ^ b_x ^ ((g16 & 1) << 1)) + ((s16 & 3) >> 1)) << 4);
    }
    // BT: B row (output column) c, k-chunk q sits at 16K + c*64 + ((q ^ ((c/4)%4)) * 16),
    // as A's rows do; fragment ni at bt16_rd + ni*1024.
    const int bt16_rd = 16384 + (wn * 128 + s16) * 64 + ((g16 ^ ((s16 >> 2) & 3)) << 4);
    // Short tiles (32x32x16): lane l covers column l%32 at k = 8*(l/32) .. +7 of a
    // 16-k sub-step, so its k-rows have bit 3 = l/32.
    const int b_c = ((g16 & 1) * 2 + ((s16 & 3) >> 1)) ^ ((g16 >> 1) << 1);
    const int b_lane = 16384 + ((g16 >> 1) * 8 + (s16 >> 2)) * 256 + (s16 & 1) * 8;

    const uint32_t lds_base = uniform((int)(uint32_t)(uintptr_t)(lds_void*)smem);
    const int G = gridDim.x;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int per_xcd = G >> 3;
    const int KT = Kd / kP4BK;
    const SplitPlan sp = split_plan(total, G, KT, part != nullptr);
    const int whole = sp.S > 1 ? sp.R * G : total;  // tiles computed in one piece
    // Work item j of this XCD is round j / per_xcd, slot j % per_xcd.  Without
    // tickets, workgroup `slot` of the XCD takes items slot, slot + per_xcd, ...;
    // with them, the XCD's workgroups claim its items in order from the XCD's
    // counter, so that a workgroup that drew short tiles takes more.  Thread 0
    // claims the next item as soon as a tile starts (the atomic's latency hides
    // under the K-loop) and passes it on after the K-loop.
    int j = slot;
    int claimed = 0;  // thread 0 only
    auto claim = [&]() {
        if (tid == 0) claimed = atomicAdd(tickets + xcd * 16, 1);
    };
    // Hands thread 0's claim to every wave through a word of the last stage.
    // The first barrier retires every read of the stages; the word is read
    // before the next tile's first in-loop barrier, and only the refill after
    // that barrier writes the last stage again.
    auto take = [&]() -> int {
        __syncthreads();
        if (tid == 0) *reinterpret_cast<volatile int*>(smem + kP4TicketOff) = claimed;
        __syncthreads();
        return uniform(*reinterpret_cast<volatile int*>(smem + kP4TicketOff));
    };
    if (tickets != nullptr) {
        claim();
        j = take();
    }
    for (;;) {
        const int round = j / per_xcd, jslot = j - round * per_xcd;
        int tile = round * G + xcd * per_xcd + jslot;
        int ks0 = 0, ksn = KT;  // K-steps of this work item
        int pslot = -1;         // split-workspace slot of a tile part
        if (tile >= whole) {
            if (sp.S == 1 || round != sp.R) break;
            const int p = xcd * per_xcd + jslot;
            if (p >= sp.Tr * sp.S) break;
            tile = whole + p / sp.S;
            const int pj = p % sp.S, q = KT / 4;
            ks0 = (pj * q / sp.S) * 4;
            ksn = ((pj + 1) * q / sp.S) * 4 - ks0;
            pslot = p;
        }
        TileGeom tg;
        if (!tile_geom_regs(sreg, NT, OUTW, rows, lane, tile, tg)) break;
        const int e = tg.e, r0 = tg.r0, rows_valid = tg.rows_valid, n0 = tg.n0;
        if (tickets != nullptr) claim();
        int j_next = j + per_xcd;
        if (rows_valid <= 0) {
            j = tickets != nullptr ? take() : j_next;
            continue;
        }

        // The tile body, instantiated per case so that neither the partial-slot
        // epilogue of the split round nor the short-tile layouts weigh on the
        // register allocation of the full tile.  MI == 0: full 256-row layout;
        // MI > 0: short tile of at most 32 * MI rows (see below).
        auto run_tile = [&](auto part_tag, auto mi_tag) {
            constexpr bool PART = decltype(part_tag)::value;
            constexpr int MI = decltype(mi_tag)::value;
            // DMA sources.  A: 16 rows of 64 bytes per KB; rows past the segment are
            // clamped to its last row.  B: 4 k-rows of one 128-column half per KB.
            // With `gather`, A is the token-ordered X (xrows rows) and
            // expert-sorted row p is read from X row gather[p] / gK, clamped
            // into [0, xrows) (page [P4] section 1: the gather fused into the
            // GEMM's loads, so the permuted copy of X is never written).
            const rsrc_t ra = make_rsrc(gather != nullptr ? A : A + (size_t)r0 * Kd);
            const int half = wave >> 1;
            const uint16_t* bmat = (DUAL && half) ? B1 : B0;
            // BT: each expert's B0 (and B1) is N x kb; the descriptor's range
            // ends at that matrix.
            const int ktb = BT ? kb / kP4BK : KT;  // first K-step read from B1
            const rsrc_t rb = BT ? make_rsrc(B0 + (size_t)e * kb * N, (uint32_t)((size_t)kb * N * 2))
                                 : make_rsrc(bmat + (size_t)e * Kd * N);
            const rsrc_t rb1 = (BT && B1 != nullptr) ? make_rsrc(B1 + (size_t)e * kb * N, (uint32_t)((size_t)kb * N * 2))
                                                     : rb;
            uint32_t a_vo[4], b_vo[4];
            #pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = (wave * 4 + i) * 16 + (lane >> 2);
                const int ch = (lane & 3) ^ ((r >> 2) & 3);
                const int rr = min(r, rows_valid - 1);
                const uint32_t arow =
                    gather != nullptr ? (uint32_t)min(max(gather[r0 + rr], 0) / gK, xrows - 1) : (uint32_t)rr;
                a_vo[i] = (arow * (uint32_t)Kd + ch * 8) * 2u;
                const int kr = (wave & 1) * 16 + i * 4 + (lane >> 4);
                const int bc = (lane & 15) ^ ((kr & 3) << 2) ^ (((kr >> 3) & 1) << 1);
                const int col = (DUAL ? n0 : n0 + half * 128) + bc * 8;
                b_vo[i] = BT ? ((uint32_t)(n0 + r) * (uint32_t)kb + ch * 8) * 2u
                             : ((uint32_t)kr * (uint32_t)N + col) * 2u;
            }
            const uint32_t b_step = (uint32_t)kP4BK * (uint32_t)N * 2u;
            // DMA number i (0..7) of K-step kt into the stage at byte offset soff:
            // i < 4 are A, the rest B.
            auto issue_one = [&](int kt, int soff, int i) {
                const uint32_t dst = lds_base + soff + (wave * 4) * 1024;
                const uint32_t ka = (uint32_t)(ks0 + kt);
                if (i < 4) dma16(ra, dst + i * 1024, a_vo[i], ka * (kP4BK * 2));
                else if constexpr (BT) {
                    const bool hi = (int)ka >= ktb;
                    dma16(hi ? rb1 : rb, dst + 16384 + (i - 4) * 1024, b_vo[i - 4],
                          (hi ? ka - (uint32_t)ktb : ka) * (kP4BK * 2));
                } else dma16(rb, dst + 16384 + (i - 4) * 1024, b_vo[i - 4], ka * b_step);
            };
            auto issue = [&](int kt, int soff) {
                #pragma unroll
                for (int i = 0; i < 8; ++i) issue_one(kt, soff, i);
            };

            if constexpr (MI == 0) {
                // acc[mi][ni]: rows mi*16.. of the wave's 128 by output columns
                // ni*16.. of its 128 (SwiGLU: ni < 4 the W1 part, ni >= 4 the W3
                // part of the same columns).  A step of K = 32 is one MFMA per
                // block, in two halves (column blocks 0..3, then 4..7), each row
                // block by row block.  Fragments are reloaded in place one half
                // ahead: B fragments 4..7 of a step under its first half, and in
                // the second half, right after row block mi's last MFMA of the
                // step, that row's A fragment of the next step, along with the
                // next step's B fragments 0..3.
                f32x4 acc[8][8];
                bf16x8 af[8], bfr[8];
                auto load_a = [&](int soff, int mi) {
                    af[mi] = *reinterpret_cast<const bf16x8*>(smem + soff + a16_rd + mi * 1024);
                };
                auto load_b = [&](int soff, int ni) {
                    if constexpr (BT) {
                        bfr[ni] = *reinterpret_cast<const bf16x8*>(smem + soff + bt16_rd + ni * 1024);
                    } else {
                        const char* pb = smem + soff + b16_rd[ni];
                        const bf16x4 h0 = lds_read_tr(pb);
                        const bf16x4 h1 = lds_read_tr(pb + 4 * 256);
                        bfr[ni] = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
                    }
                };
                // The four MFMAs of row block mi in half h (column blocks 4h .. 4h+3);
                // with z the accumulators start from zero (the first K-step).
                auto mfma_row = [&](int h, int mi, bool z) {
                    #pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (z) mfma16_first(acc[mi][4 * h + j], bfr[4 * h + j], af[mi]);
                        else mfma16(acc[mi][4 * h + j], bfr[4 * h + j], af[mi]);
                    }
                };

                // Prologue (ksn is a multiple of 4 here): K-steps 0..3 in flight, wait for step 0.
                issue(0, 0);
                issue(1, kP4Stage);
                issue(2, 2 * kP4Stage);
                issue(3, 3 * kP4Stage);
                __asm__ volatile("s_waitcnt vmcnt(24)" ::: "memory");
                __syncthreads();
                #pragma unroll
                for (int mi = 0; mi < 8; ++mi) load_a(0, mi);
                #pragma unroll
                for (int ni = 0; ni < 4; ++ni) load_b(0, ni);

                // One K-step per loop iteration: unrolled, the reloads in place
                // defeat the register allocator's coalescing of the accumulators.
                int s_cur = 0;  // byte offset of step kt's stage
                auto kstep = [&](int kt, auto first_tag) {
                    constexpr bool Z = decltype(first_tag)::value;
                    {
                        const int s_nxt = s_cur == (kP4Stages - 1) * kP4Stage ? 0 : s_cur + kP4Stage;
                        const int s_old = s_cur == 0 ? (kP4Stages - 1) * kP4Stage : s_cur - kP4Stage;
                        // Step boundary: own DMA of step kt+1 done (16 younger ones may
                        // fly), then the barrier.  No wait for this wave's LDS reads: the
                        // reads still in flight are of step kt+1's stage, and the stage
                        // refilled below (step kt-1's) was last read by fragments that
                        // step kt-1's MFMAs have consumed.
                        __builtin_amdgcn_sched_barrier(0);
                        __asm__ volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
                        // Refill the stage of step kt-1 with step kt+4: one DMA before
                        // each of the first four row blocks of each half, so that a DMA
                        // held up by a full address queue delays few MFMAs.
                        const int kn = min(kt + 4, ksn - 1);
                        #pragma unroll
                        for (int mi = 0; mi < 8; ++mi) {
                            if (mi < 4) issue_one(kn, s_old, mi);
                            mfma_row(0, mi, Z);
                            if (mi < 4) load_b(s_cur, 4 + mi);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        #pragma unroll
                        for (int mi = 0; mi < 8; ++mi) {
                            if (mi < 4) issue_one(kn, s_old, 4 + mi);
                            mfma_row(1, mi, Z);
                            load_a(s_nxt, mi);
                            if (mi >= 2 && mi < 6) load_b(s_nxt, mi - 2);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        s_cur = s_nxt;
                    }
                };
                kstep(0, std::true_type{});
                for (int kt = 1; kt < ksn; ++kt) kstep(kt, std::false_type{});
                mfma16_drain(acc);
                // The clamped refills of the last steps are still in flight.
                __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
                // Every wave is done reading the stages (the staged epilogue below
                // reuses them).
                if (tickets != nullptr) j_next = take();
                else __syncthreads();

                #pragma unroll
                for (int sl = 0; sl < 4; ++sl) {  // 32-row slices: row blocks 2sl, 2sl+1
                    if constexpr (BWD && DUAL) {
                        store_rows_lds_raw(acc, sl, smem, C, (size_t)rows * N, r0, rows_valid, n0, N, wave, wm, wn);
                    } else if constexpr (BWD) {
                        if (sl == 0) bwd_rows_lds(acc, smem, r0, rows_valid, n0, N, wave, wm, wn, bwd);
                    } else if constexpr (PART) {
                        f32x4* dst = reinterpret_cast<f32x4*>(part + (size_t)pslot * kPartFloats);
                        const int ln = __lane_id();
                        #pragma unroll
                        for (int mm = 0; mm < 2; ++mm)
                            #pragma unroll
                            for (int ni = 0; ni < 8; ++ni)
                                dst[part_index(wave, 2 * sl + mm, ni, ln)] = acc[2 * sl + mm][ni];
                    } else {
                        store_rows_lds<DUAL>(acc, sl, smem, C, r0, rows_valid, n0, N, wave, wm, wn);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                // Short tile: every row sits in the first 32 * MI.  The four waves
                // share those rows and each takes a quarter of the columns (the W1
                // and W3 halves of 32 output columns for the SwiGLU GEMM, 64
                // columns otherwise), so only row slices that hold rows are
                // multiplied.  Stages, DMA, waits and barriers are the full tile's.
                int sa_rd[2], sb_rd[2];
                #pragma unroll
                for (int ks = 0; ks < 2; ++ks) sa_rd[ks] = l32 * 64 + (((ks * 2 + lh) ^ ((l32 >> 2) & 3)) << 4);
                #pragma unroll
                for (int ni = 0; ni < 2; ++ni) {
                    const int sh = DUAL ? ni : (wave >> 1);
                    const int nn = DUAL ? wave * 32 : (wave & 1) * 64 + ni * 32;
                    sb_rd[ni] = b_lane + sh * 8192 + ((((nn >> 3) ^ b_x) + b_c) << 4);
                }
                // BT: this wave's output columns wave*64 + ni*32 are B rows, read as A's.
                int sbt_rd[2];
                #pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    sbt_rd[ks] = 16384 + (wave * 64 + l32) * 64 + (((ks * 2 + lh) ^ ((l32 >> 2) & 3)) << 4);
                f32x16 acc[MI][2];
                #pragma unroll
                for (int mi = 0; mi < MI; ++mi)
                    #pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
                        #pragma unroll
                        for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.0f;
                bf16x8 af[2][MI], bfr[2][2];
                auto load_frags = [&](int soff, int ks, int buf) {
                    const char* sa = smem + soff + sa_rd[ks];
                    #pragma unroll
                    for (int mi = 0; mi < MI; ++mi) af[buf][mi] = *reinterpret_cast<const bf16x8*>(sa + mi * 32 * 64);
                    #pragma unroll
                    for (int ni = 0; ni < 2; ++ni) {
                        if constexpr (BT) {
                            bfr[buf][ni] = *reinterpret_cast<const bf16x8*>(smem + soff + sbt_rd[ks] + ni * 32 * 64);
                        } else {
                            const char* pb = smem + soff + sb_rd[ni] + ks * 16 * 256;
                            const bf16x4 h0 = lds_read_tr(pb);
                            const bf16x4 h1 = lds_read_tr(pb + 4 * 256);
                            bfr[buf][ni] = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
                        }
                    }
                };
                auto mfma = [&](int buf) {
                    #pragma unroll
                    for (int mi = 0; mi < MI; ++mi)
                        #pragma unroll
                        for (int ni = 0; ni < 2; ++ni)
                            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[buf][ni], af[buf][mi], acc[mi][ni], 0, 0, 0);
                };
                issue(0, 0);
                issue(1, kP4Stage);
                issue(2, 2 * kP4Stage);
                issue(3, 3 * kP4Stage);
                __asm__ volatile("s_waitcnt vmcnt(24)" ::: "memory");
                __syncthreads();
                load_frags(0, 0, 0);
                int s_cur = 0;
                for (int kt = 0; kt < ksn; ++kt) {
                    const int s_nxt = s_cur == (kP4Stages - 1) * kP4Stage ? 0 : s_cur + kP4Stage;
                    const int s_old = s_cur == 0 ? (kP4Stages - 1) * kP4Stage : s_cur - kP4Stage;
                    __builtin_amdgcn_sched_barrier(0);
                    __asm__ volatile("s_waitcnt vmcnt(16)" ::: "memory");
                    __syncthreads();
                    issue(min(kt + 4, ksn - 1), s_old);
                    load_frags(s_cur, 1, 1);
                    mfma(0);
                    load_frags(s_nxt, 0, 0);
                    mfma(1);
                    s_cur = s_nxt;
                }
                __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
                if (tickets != nullptr) j_next = take();
                #pragma unroll
                for (int mi = 0; mi < MI; ++mi) {
                    if constexpr (BWD && DUAL) store_rows_short_raw(acc[mi], mi, C, (size_t)rows * N, r0, rows_valid, n0, N, wave);
                    else if constexpr (BWD) bwd_rows_short(acc[mi], mi, r0, rows_valid, n0, N, wave, bwd);
                    else store_rows_short<DUAL>(acc[mi], mi, C, r0, rows_valid, n0, N, wave);
                }
            }
        };
        using Full = std::integral_constant<int, 0>;
        if (pslot >= 0) {
            if constexpr (!BWD) run_tile(std::true_type{}, Full{});  // (no split tail with the fused epilogue)
        }
        else if (rows_valid <= 32) run_tile(std::false_type{}, std::integral_constant<int, 1>{});
        else if (rows_valid <= 64) run_tile(std::false_type{}, std::integral_constant<int, 2>{});
        else if (rows_valid <= 128) run_tile(std::false_type{}, std::integral_constant<int, 4>{});
        else run_tile(std::false_type{}, Full{});
        j = j_next;
    }
}

// Expert-weight gradients on the pipelined kernel's K-loop (page [P4] section
// 2.2: dW1 = X^T dH1, dW3 = X^T dH3, dW2 = (w act)^T dY, each over one
// expert's rows).  For expert e with cnt = counts[e] rows starting at
// offsets[e]: C[e] (M x N, fp32, row-major) = P_e^T Q_e, P_e the rows of P
// (row stride ldp) and Q_e those of Q (row stride ldq, from column qoff).
// The reduction runs over the rows, 32 per K-step, so both operands arrive
// with K outermost: each is staged as the forward kernel stages its weights
// (32 k-rows of two 128-column halves, XOR-swizzled by 16-byte piece) and
// read with the transposing LDS read.  Rows past cnt read as zero: each
// operand's buffer descriptor ends at the expert's last row, and the whole
// offset goes in the range-checked VGPR operand.  An expert's rows are
// clamped to the `rows` rows the operands hold, whatever counts and offsets
// say.  One 256 x 256 tile per work item, four waves of 128 x 128; a tile of
// an expert without rows skips the K-loop and stores zeros.
__global__ __launch_bounds__(kThreads, 1) void dw_p4_kernel(
    const uint16_t* __restrict__ P, int ldp, const uint16_t* __restrict__ Q, int ldq, int qoff,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets, int E, int M, int N, int rows,
    float* __restrict__ C) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = uniform(tid / kWave);
    const int wm = wave >> 1, wn = wave & 1;
    const int g16 = lane >> 4, s16 = lane & 15;
    // Fragment reads (v_mfma_f32_16x16x32_bf16, as the forward kernel's whole
    // tiles): column c of half h of an operand staged at X (P at 0, Q at 16K)
    // sits at X + h*8K + k*256 + ((c/8) ^ 4*(k%4) ^ 2*((k/8)%2)) * 16 + (c%8)*2;
    // lane l reads column l%16 of a 16-column block at k = 8*(l/16) .. +7.
    const int b_x = (s16 >> 2) << 2;
    const int rd_lane = (g16 * 8 + (s16 >> 2)) * 256 + (s16 & 1) * 8;
    int p_rd[8], q_rd[8];
    #pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int piece = ((((i * 16) >> 3) ^ b_x ^ ((g16 & 1) << 1)) + ((s16 & 3) >> 1)) << 4;
        p_rd[i] = rd_lane + wm * 8192 + piece;
        q_rd[i] = 16384 + rd_lane + wn * 8192 + piece;
    }
    const uint32_t lds_base = uniform((int)(uint32_t)(uintptr_t)(lds_void*)smem);
    const int G = gridDim.x;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int per_xcd = G >> 3;
    const int MT = M / 256, NT = N / 256;
    const int total = E * MT * NT;
    // Work item j of this XCD: round j / per_xcd, slot j % per_xcd, as in the
    // forward kernel, so that an XCD's workgroups share P panels in L2.
    for (int j = slot;; j += per_xcd) {
        const int round = j / per_xcd, jslot = j - round * per_xcd;
        const int tile = round * G + xcd * per_xcd + jslot;
        if (tile >= total) break;
        const int e = tile / (MT * NT);
        const int rem = tile - e * MT * NT;
        const int m0 = (rem / NT) * 256, n0 = (rem - (rem / NT) * NT) * 256;
        const int r0 = min(max(uniform(offsets[e]), 0), rows);
        const int cnt = min(max(uniform(counts[e]), 0), rows - r0);
        const int ksn = (cnt + 127) / 128 * 4;  // a multiple of 4 K-steps; 0 for an expert without rows
        const rsrc_t rp = make_rsrc(P + (size_t)r0 * ldp, (uint32_t)cnt * (uint32_t)ldp * 2u);
        const rsrc_t rq = make_rsrc(Q + (size_t)r0 * ldq + qoff, (uint32_t)cnt * (uint32_t)ldq * 2u);
        uint32_t p_vo[4], q_vo[4];
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kr = (wave & 1) * 16 + i * 4 + (lane >> 4);
            const int col = (wave >> 1) * 128 + (((lane & 15) ^ ((kr & 3) << 2) ^ (((kr >> 3) & 1) << 1)) << 3);
            p_vo[i] = ((uint32_t)kr * (uint32_t)ldp + (uint32_t)(m0 + col)) * 2u;
            q_vo[i] = ((uint32_t)kr * (uint32_t)ldq + (uint32_t)(n0 + col)) * 2u;
        }
        const uint32_t p_step = 64u * (uint32_t)ldp, q_step = 64u * (uint32_t)ldq;
        auto issue_one = [&](int kt, int soff, int i) {
            const uint32_t dst = lds_base + soff + wave * 4096;
            if (i < 4) dma16(rp, dst + i * 1024, p_vo[i] + (uint32_t)kt * p_step, 0);
            else dma16(rq, dst + 16384 + (i - 4) * 1024, q_vo[i - 4] + (uint32_t)kt * q_step, 0);
        };
        auto issue = [&](int kt, int soff) {
            #pragma unroll
            for (int i = 0; i < 8; ++i) issue_one(kt, soff, i);
        };
        // acc[mi][ni]: rows (M) mi*16.. and columns (N) ni*16.. of the wave's
        // 128 x 128 quadrant; the K-loop is the forward kernel's whole-tile loop.
        f32x4 acc[8][8];
        if (ksn > 0) {  // (uniform over the workgroup: one expert per tile)
            bf16x8 af[8], bfr[8];
            auto load_p = [&](int soff, int mi) {
                const char* pa = smem + soff + p_rd[mi];
                af[mi] = __builtin_shufflevector(lds_read_tr(pa), lds_read_tr(pa + 4 * 256), 0, 1, 2, 3, 4, 5, 6, 7);
            };
            auto load_q = [&](int soff, int ni) {
                const char* pb = smem + soff + q_rd[ni];
                bfr[ni] = __builtin_shufflevector(lds_read_tr(pb), lds_read_tr(pb + 4 * 256), 0, 1, 2, 3, 4, 5, 6, 7);
            };
            auto mfma_row = [&](int h, int mi, bool z) {
                #pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (z) mfma16_first(acc[mi][4 * h + j], bfr[4 * h + j], af[mi]);
                    else mfma16(acc[mi][4 * h + j], bfr[4 * h + j], af[mi]);
                }
            };
            issue(0, 0);
            issue(1, kP4Stage);
            issue(2, 2 * kP4Stage);
            issue(3, 3 * kP4Stage);
            __asm__ volatile("s_waitcnt vmcnt(24)" ::: "memory");
            __syncthreads();
            #pragma unroll
            for (int mi = 0; mi < 8; ++mi) load_p(0, mi);
            #pragma unroll
            for (int ni = 0; ni < 4; ++ni) load_q(0, ni);
            int s_cur = 0;
            auto kstep = [&](int kt, auto first_tag) {
                constexpr bool Z = decltype(first_tag)::value;
                const int s_nxt = s_cur == (kP4Stages - 1) * kP4Stage ? 0 : s_cur + kP4Stage;
                const int s_old = s_cur == 0 ? (kP4Stages - 1) * kP4Stage : s_cur - kP4Stage;
                // Step boundary as in the forward kernel: own DMA of step kt+1 done,
                // then a bare barrier (reads in flight are of step kt+1's stage).
                __builtin_amdgcn_sched_barrier(0);
                __asm__ volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
                const int kn = min(kt + 4, ksn - 1);
                #pragma unroll
                for (int mi = 0; mi < 8; ++mi) {
                    if (mi < 4) issue_one(kn, s_old, mi);
                    mfma_row(0, mi, Z);
                    if (mi < 4) load_q(s_cur, 4 + mi);
                    __builtin_amdgcn_sched_barrier(0);
                }
                #pragma unroll
                for (int mi = 0; mi < 8; ++mi) {
                    if (mi < 4) issue_one(kn, s_old, 4 + mi);
                    mfma_row(1, mi, Z);
                    load_p(s_nxt, mi);
                    if (mi >= 2 && mi < 6) load_q(s_nxt, mi - 2);
                    __builtin_amdgcn_sched_barrier(0);
                }
                s_cur = s_nxt;
            };
            kstep(0, std::true_type{});
            for (int kt = 1; kt < ksn; ++kt) kstep(kt, std::false_type{});
            mfma16_drain(acc);
            __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            // Every wave is done reading the stages before the next tile refills them.
            __syncthreads();
        } else {
            #pragma unroll
            for (int mi = 0; mi < 8; ++mi)
                #pragma unroll
                for (int ni = 0; ni < 8; ++ni) acc[mi][ni] = f32x4{};
        }
        // acc[mi][ni] element v of lane l: row wm*128 + mi*16 + l%16, column
        // wn*128 + ni*16 + 4*(l/16) + v of the tile.
        float* cbase = C + ((size_t)e * M + m0 + wm * 128 + s16) * N + n0 + wn * 128 + 4 * g16;
        #pragma unroll
        for (int mi = 0; mi < 8; ++mi)
            #pragma unroll
            for (int ni = 0; ni < 8; ++ni)
                *reinterpret_cast<f32x4*>(cbase + (size_t)(mi * 16) * N + ni * 16) = acc[mi][ni];
    }
}

// Finishes the split tiles of the pipelined kernel launched with G workgroups:
// adds each tile's S partial slots in slot order and runs the epilogue.
template <bool DUAL>
__global__ __launch_bounds__(kThreads) void ffn_split_fixup(const float* __restrict__ part, uint16_t* __restrict__ C,
                                                            const int32_t* __restrict__ counts,
                                                            const int32_t* __restrict__ offsets, int E, int Kd, int N,
                                                            int rows, int G) {
    constexpr int OUTW = DUAL ? 128 : 256;
    const int NT = N / OUTW;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, lh = lane >> 5;
    int total = 0, first = 0;
    sched_lookup(counts, E, NT, rows, lane, -1, &first, &total);
    total = uniform(total);
    const SplitPlan sp = split_plan(total, G, Kd / kP4BK, true);
    if (sp.S == 1) return;
    // one work unit per (split tile, 32-row slice of every wave's quadrant)
    for (int u = blockIdx.x; u < sp.Tr * 4; u += gridDim.x) {
        const int i = u >> 2, sl = u & 3;
        TileGeom tg;
        if (!tile_geom(counts, offsets, E, NT, OUTW, rows, lane, sp.R * G + i, tg)) return;
        if (tg.rows_valid <= 0) continue;
        const f32x4* src = reinterpret_cast<const f32x4*>(part + (size_t)i * sp.S * kPartFloats);
        f32x4 acc[2][8];
        #pragma unroll
        for (int mm = 0; mm < 2; ++mm)
            #pragma unroll
            for (int ni = 0; ni < 8; ++ni) acc[mm][ni] = f32x4{};
        for (int j = 0; j < sp.S; ++j) {  // parts in slot order
            f32x4 v[2][8];
            #pragma unroll
            for (int mm = 0; mm < 2; ++mm)
                #pragma unroll
                for (int ni = 0; ni < 8; ++ni)
                    v[mm][ni] = src[(size_t)j * (kPartFloats / 4) + part_index(wave, 2 * sl + mm, ni, lane)];
            #pragma unroll
            for (int mm = 0; mm < 2; ++mm)
                #pragma unroll
                for (int ni = 0; ni < 8; ++ni)
                    #pragma unroll
                    for (int c = 0; c < 4; ++c) acc[mm][ni][c] += v[mm][ni][c];
        }
        store_rows<DUAL>(acc, sl, C, tg.r0, tg.rows_valid, tg.n0, N, wm, wn);
    }
}

// The router projection on the SwiGLU GEMM's kernel: A = X (T rows, one
// "expert"), B0 = hi and B1 = lo, the two bf16 terms of the fp32 router
// weights ([d, E], E columns).  The launch has fewer than half as many tiles as
// workgroups, so every tile is split along K and the kernel only leaves fp32
// partial tiles.  This adds a tile's slots in slot order, for each of its
// columns the hi part and the lo part, and writes
// logits[t, c] = (hi sum + lo sum) + bias[c] as fp32.
__global__ __launch_bounds__(kThreads) void router_fixup(const float* __restrict__ part, float* __restrict__ logits,
                                                         const float* __restrict__ bias,
                                                         const int32_t* __restrict__ counts,
                                                         const int32_t* __restrict__ offsets, int Kd, int N,
                                                         int rows, int G) {
    constexpr int OUTW = 128;
    const int NT = N / OUTW;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int wm = wave >> 1, wn = wave & 1;
    const int s16 = lane & 15, g16 = lane >> 4;
    int total = 0, first = 0;
    sched_lookup(counts, 1, NT, rows, lane, -1, &first, &total);
    total = uniform(total);
    const SplitPlan sp = split_plan(total, G, Kd / kP4BK, true);
    if (sp.R != 0 || sp.S < 2) return;  // not a fully split launch (the host rules it out)
    for (int u = blockIdx.x; u < sp.Tr * 4; u += gridDim.x) {
        const int i = u >> 2, sl = u & 3;
        TileGeom tg;
        if (!tile_geom(counts, offsets, 1, NT, OUTW, rows, lane, i, tg)) return;
        if (tg.rows_valid <= 0) continue;
        const f32x4* src = reinterpret_cast<const f32x4*>(part + (size_t)i * sp.S * kPartFloats);
        f32x4 acc[2][8];
        #pragma unroll
        for (int mm = 0; mm < 2; ++mm)
            #pragma unroll
            for (int ni = 0; ni < 8; ++ni) acc[mm][ni] = f32x4{};
        for (int j = 0; j < sp.S; ++j) {  // parts in slot order
            #pragma unroll
            for (int mm = 0; mm < 2; ++mm)
                #pragma unroll
                for (int ni = 0; ni < 8; ++ni) {
                    const f32x4 v = src[(size_t)j * (kPartFloats / 4) + part_index(wave, 2 * sl + mm, ni, lane)];
                    #pragma unroll
                    for (int c = 0; c < 4; ++c) acc[mm][ni][c] += v[c];
                }
        }
        // lane l: row l%16 of block mm, columns ni*16 + 4*(l/16) .. +3 of the
        // wave's 64 (ni < 4 the hi part, ni + 4 the lo part of the same columns)
        #pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
            const int m = wm * 128 + sl * 32 + mm * 16 + s16;
            if (m < tg.rows_valid) {
                float* orow = logits + (size_t)(tg.r0 + m) * N;
                #pragma unroll
                for (int ni = 0; ni < 4; ++ni) {
                    const int c = tg.n0 + wn * 64 + ni * 16 + 4 * g16;
                    f32x4 o;
                    #pragma unroll
                    for (int q = 0; q < 4; ++q)
                        o[q] = (acc[mm][ni][q] + acc[mm][ni + 4][q]) + (bias != nullptr ? bias[c + q] : 0.0f);
                    *reinterpret_cast<f32x4*>(orow + c) = o;
                }
            }
        }
    }
}

// Clears the claim counters before a launch of the pipelined kernel.
__global__ void zero_ints(int* __restrict__ p, int n) {
    if ((int)threadIdx.x < n) p[threadIdx.x] = 0;
}

// fp32 tile kernel (plain FMA): block tile 64 x 64 x 16, each thread 4 x 4 outputs.
template <bool DUAL>
__global__ __launch_bounds__(kThreads) void ffn_f32_kernel(const float* __restrict__ A,
                                                           const float* __restrict__ B0,
                                                           const float* __restrict__ B1,
                                                           float* __restrict__ C,
                                                           const int32_t* __restrict__ counts,
                                                           const int32_t* __restrict__ offsets, int E,
                                                           int Kd, int N, int rows) {
    constexpr int BM = 64, BN = 64, BK = 16;
    constexpr int NB = DUAL ? 2 : 1;
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs[NB][BK][BN + 4];
    __shared__ int s_start[257];
    __shared__ int s_tmp[256];
    const int NT = N / BN;
    build_schedule<BM>(counts, E, NT, rows, s_start, s_tmp);
    const int total = s_start[E];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;

    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const int e = find_expert(s_start, E, tile);
        const int cnt = min(max(counts[e], 0), rows);
        const int mt = (cnt + BM - 1) / BM;
        const int local = tile - s_start[e];
        const int m_tile = local % mt;
        const int n_tile = local / mt;
        const int r0 = offsets[e] + m_tile * BM;
        // rows of this tile that exist; never past the end of A/C whatever counts/offsets hold
        const int rows_valid = (r0 < 0 || r0 >= rows) ? 0 : min(min(BM, cnt - m_tile * BM), rows - r0);
        const size_t row0 = (size_t)max(r0, 0);
        const int n0 = n_tile * BN;
        const float* Bp[2] = {B0 + (size_t)e * Kd * N, DUAL ? B1 + (size_t)e * Kd * N : nullptr};
        float acc[NB][4][4];
        #pragma unroll
        for (int m = 0; m < NB; ++m)
            #pragma unroll
            for (int i = 0; i < 4; ++i)
                #pragma unroll
                for (int j = 0; j < 4; ++j) acc[m][i][j] = 0.0f;
        for (int k0 = 0; k0 < Kd; k0 += BK) {
            __syncthreads();
            #pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = tid + kThreads * i;
                const int r = c >> 4, kk = c & 15;
                As[kk][r] = (r < rows_valid) ? A[(row0 + r) * Kd + k0 + kk] : 0.0f;
            }
            #pragma unroll
            for (int m = 0; m < NB; ++m)
                #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = tid + kThreads * i;
                    const int kk = c >> 6, nn = c & 63;
                    Bs[m][kk][nn] = Bp[m][(size_t)(k0 + kk) * N + n0 + nn];
                }
            __syncthreads();
            #pragma unroll
            for (int kk = 0; kk < BK; ++kk) {
                float a[4], b[NB][4];
                #pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
                #pragma unroll
                for (int m = 0; m < NB; ++m)
                    #pragma unroll
                    for (int j = 0; j < 4; ++j) b[m][j] = Bs[m][kk][tx + 16 * j];
                #pragma unroll
                for (int m = 0; m < NB; ++m)
                    #pragma unroll
                    for (int i = 0; i < 4; ++i)
                        #pragma unroll
                        for (int j = 0; j < 4; ++j) acc[m][i][j] = fmaf(a[i], b[m][j], acc[m][i][j]);
            }
        }
        #pragma unroll
        for (int i = 0; i < 4; ++i)
            #pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = ty + 16 * i;
                if (row < rows_valid) {
                    float v = acc[0][i][j];
                    if (DUAL) {
                        const float h3 = acc[NB - 1][i][j];
                        v = v / (1.0f + expf(-v)) * h3;
                    }
                    C[(row0 + row) * N + n0 + tx + 16 * j] = v;
                }
            }
    }
}

}  // namespace

// The pipelined bf16 kernel needs 256-wide down-projection tiles and K in
// multiples of 128 for both GEMMs, and addresses one expert's weight matrix
// with 32-bit buffer offsets below the descriptor's 2^31-byte range.
static bool ffn_pipelined_ok(int d, int n) {
    return d % 256 == 0 && n % 128 == 0 && (long long)d * n * 2 < (1LL << 31);
}

bool ffn_raw_ok(int dtype, int d, int n) { return dtype == 1 && ffn_pipelined_ok(d, n); }

// Gathered loads address X with 32-bit byte offsets.
bool ffn_gather_ok(int dtype, int T, int d, int n) {
    return dtype == 1 && ffn_pipelined_ok(d, n) && (long long)T * d * 2 < (1LL << 31);
}

static int ffn_grid() { return (device_cu_count() / 8) * 8; }

// Split slots for every workgroup, then two sets of claim counters (the
// SwiGLU GEMM's, then the down GEMM's).
size_t ffn_split_bytes(int dtype, int d, int n) {
    return (dtype == 1 && ffn_pipelined_ok(d, n))
               ? (size_t)ffn_grid() * kPartFloats * sizeof(float) + 2 * kTicketInts * sizeof(int)
               : 0;
}

int* ffn_tickets(float* part) { return part ? reinterpret_cast<int*>(part + (size_t)ffn_grid() * kPartFloats) : nullptr; }
int ffn_ticket_ints() { return 2 * kTicketInts; }

// One pipelined GEMM (SwiGLU or plain), then the fixup of its split tail.
// BWD: the SwiGLU-backward epilogue (`bwd`) instead of a store of C; no split.
template <bool DUAL, bool BT = false, bool BWD = false>
static hipError_t launch_pipelined(const uint16_t* A, const uint16_t* B0, const uint16_t* B1, uint16_t* C,
                                   const int32_t* counts, const int32_t* offsets, int E, int Kd, int N, int rows,
                                   float* part, bool tickets_zeroed, const int32_t* gather, int gK, int xrows,
                                   hipStream_t s, int kb = 0, const BwdEpi& bwd = BwdEpi{}) {
    if (BWD && part != nullptr) return hipErrorInvalidValue;
    const hipError_t aerr = hipFuncSetAttribute((const void*)ffn_p4_kernel<DUAL, BT, BWD>,
                                                hipFuncAttributeMaxDynamicSharedMemorySize, kP4Lds);
    if (aerr != hipSuccess) return aerr;
    const int G = ffn_grid();
    int* tickets = part != nullptr ? ffn_tickets(part) + (DUAL ? 0 : kTicketInts) : nullptr;
    if (tickets != nullptr && !tickets_zeroed)
        hipLaunchKernelGGL(zero_ints, dim3(1), dim3(kTicketInts), 0, s, tickets, kTicketInts);
    hipLaunchKernelGGL((ffn_p4_kernel<DUAL, BT, BWD>), dim3(G), dim3(kThreads), kP4Lds, s, A, B0, B1, C, counts,
                       offsets, E, Kd, N, rows, part, tickets, gather, gK, xrows, kb, bwd);
    if (part != nullptr)
        hipLaunchKernelGGL(ffn_split_fixup<DUAL>, dim3(G), dim3(kThreads), 0, s, part, C, counts, offsets, E, Kd, N,
                           rows, G);
    return hipGetLastError();
}

// Step 4a: Act = SiLU(Xp W1) * (Xp W3).
hipError_t launch_ffn_up(const void* Xp, const void* W1, const void* W3, int dtype, int rows, int d, int E,
                         int n, const int32_t* counts, const int32_t* offsets, void* Act, float* part,
                         bool tickets_zeroed, hipStream_t s, const int32_t* gather, int gK, int xrows) {
    const int cus = device_cu_count();
    const bool pipelined = dtype == 1 && ffn_pipelined_ok(d, n);
    // Only the pipelined kernel gathers; the others would index the
    // token-ordered X by expert-sorted row, past its end.
    if (gather != nullptr && !(pipelined && gK >= 1 && xrows >= 1 && ffn_gather_ok(dtype, xrows, d, n)))
        return hipErrorInvalidValue;
    if (pipelined)
        return launch_pipelined<true>(static_cast<const uint16_t*>(Xp), static_cast<const uint16_t*>(W1),
                                      static_cast<const uint16_t*>(W3), static_cast<uint16_t*>(Act), counts,
                                      offsets, E, d, n, rows, part, tickets_zeroed, gather, gK, xrows, s);
    if (dtype == 1) {
        hipLaunchKernelGGL(ffn_bf16_kernel<true>, dim3(cus * 2), dim3(kThreads), 0, s,
                           static_cast<const uint16_t*>(Xp), static_cast<const uint16_t*>(W1),
                           static_cast<const uint16_t*>(W3), static_cast<uint16_t*>(Act), counts, offsets, E, d,
                           n, rows);
    } else {
        hipLaunchKernelGGL(ffn_f32_kernel<true>, dim3(cus * 2), dim3(kThreads), 0, s,
                           static_cast<const float*>(Xp), static_cast<const float*>(W1),
                           static_cast<const float*>(W3), static_cast<float*>(Act), counts, offsets, E, d, n,
                           rows);
    }
    return hipGetLastError();
}

// The backward's pre-activations in one launch: H1 = Xp W1 into H and
// H3 = Xp W3 into H + rows * n (bf16, whole tiles in one piece: no split).
hipError_t launch_ffn_up_raw(const void* Xp, const void* W1, const void* W3, int rows, int d, int E, int n,
                             const int32_t* counts, const int32_t* offsets, void* H, hipStream_t s) {
    if (!ffn_pipelined_ok(d, n)) return hipErrorInvalidValue;
    return launch_pipelined<true, false, true>(static_cast<const uint16_t*>(Xp), static_cast<const uint16_t*>(W1),
                                               static_cast<const uint16_t*>(W3), static_cast<uint16_t*>(H), counts,
                                               offsets, E, d, n, rows, nullptr, false, nullptr, 1, 1, s);
}

// The router projection as a fully split SwiGLU-kernel launch (see
// router_fixup): bf16 X with d % 256 == 0, E % 128 == 0, and at most G/2 tiles
// of 256 tokens x 128 experts, so that every tile is split in at least two.
// Only for d >= 4096: the parts' prologues and epilogues and the fixup's pass
// over the fp32 slots cost about 25 us, which a shorter K does not pay back
// against the register-tiled kernel.
bool router_gemm_ok(int T, int d, int E) {
    if (T < 1 || d < 4096 || !ffn_pipelined_ok(d, E) || (long long)T * d * 2 >= (1LL << 31)) return false;
    const long long tiles = ((long long)T + kBM256 - 1) / kBM256 * (E / 128);
    const int G = ffn_grid();
    return tiles * 2 <= G && d / kP4BK / 4 >= 2;
}

hipError_t launch_router_gemm(const uint16_t* X, const uint16_t* hi, const uint16_t* lo, int T, int d, int E,
                              const int32_t* counts, const int32_t* offsets, const float* bias, float* logits,
                              float* part, bool tickets_zeroed, hipStream_t s) {
    if (!router_gemm_ok(T, d, E) || part == nullptr) return hipErrorInvalidValue;
    const hipError_t aerr = hipFuncSetAttribute((const void*)ffn_p4_kernel<true, false, false>,
                                                hipFuncAttributeMaxDynamicSharedMemorySize, kP4Lds);
    if (aerr != hipSuccess) return aerr;
    const int G = ffn_grid();
    int* tickets = ffn_tickets(part);
    if (!tickets_zeroed) hipLaunchKernelGGL(zero_ints, dim3(1), dim3(kTicketInts), 0, s, tickets, kTicketInts);
    // C is never written: every work item is a split part.
    hipLaunchKernelGGL((ffn_p4_kernel<true, false, false>), dim3(G), dim3(kThreads), kP4Lds, s, X, hi, lo,
                       static_cast<uint16_t*>(nullptr), counts, offsets, 1, d, E, T, part, tickets,
                       static_cast<const int32_t*>(nullptr), 1, T, 0, BwdEpi{});
    hipLaunchKernelGGL(router_fixup, dim3(G), dim3(kThreads), 0, s, part, logits, bias, counts, offsets, d, E, T, G);
    return hipGetLastError();
}

// Step 4b: Y = Act W2.
hipError_t launch_ffn_down(const void* Act, const void* W2, int dtype, int rows, int d, int E, int n,
                           const int32_t* counts, const int32_t* offsets, void* Y, float* part,
                           bool tickets_zeroed, hipStream_t s) {
    const int cus = device_cu_count();
    if (dtype == 1 && ffn_pipelined_ok(d, n))
        return launch_pipelined<false>(static_cast<const uint16_t*>(Act), static_cast<const uint16_t*>(W2),
                                       static_cast<const uint16_t*>(nullptr), static_cast<uint16_t*>(Y), counts,
                                       offsets, E, n, d, rows, part, tickets_zeroed, nullptr, 1, 1, s);
    if (dtype == 1) {
        hipLaunchKernelGGL(ffn_bf16_kernel<false>, dim3(cus * 2), dim3(kThreads), 0, s,
                           static_cast<const uint16_t*>(Act), static_cast<const uint16_t*>(W2),
                           static_cast<const uint16_t*>(nullptr), static_cast<uint16_t*>(Y), counts, offsets, E,
                           n, d, rows);
    } else {
        hipLaunchKernelGGL(ffn_f32_kernel<false>, dim3(cus * 2), dim3(kThreads), 0, s,
                           static_cast<const float*>(Act), static_cast<const float*>(W2),
                           static_cast<const float*>(nullptr), static_cast<float*>(Y), counts, offsets, E, n, d,
                           rows);
    }
    return hipGetLastError();
}

// The kernel numbers its 256 x 256 tiles with an int, and a workgroup's last
// tile index (before it finds no more work) reaches past the tile count by up
// to one grid.
bool dw_p4_ok(int dtype, int E, int M, int N, int rows, int ldp, int ldq) {
    const long long ld = ldp > ldq ? ldp : ldq;
    return dtype == 1 && M % 256 == 0 && N % 256 == 0 && ldp % 8 == 0 && ldq % 8 == 0 &&
           ((long long)rows + 128) * ld * 2 < (1LL << 31) &&
           (long long)E * (M / 256) * (N / 256) + ffn_grid() < (1LL << 31);
}

hipError_t launch_dw_p4(const void* P, int ldp, const void* Q, int ldq, int qoff, const int32_t* counts,
                        const int32_t* offsets, int E, int M, int N, int rows, float* dW, hipStream_t s) {
    if (!dw_p4_ok(1, E, M, N, rows, ldp, ldq) || qoff % 8 != 0 || qoff + N > ldq) return hipErrorInvalidValue;
    const hipError_t aerr =
        hipFuncSetAttribute((const void*)dw_p4_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kP4Lds);
    if (aerr != hipSuccess) return aerr;
    hipLaunchKernelGGL(dw_p4_kernel, dim3(ffn_grid()), dim3(kThreads), kP4Lds, s, static_cast<const uint16_t*>(P),
                       ldp, static_cast<const uint16_t*>(Q), ldq, qoff, counts, offsets, E, M, N, rows, dW);
    return hipGetLastError();
}

bool ffn_bt_ok(int dtype, int N, int Kd, int kb) {
    return dtype == 1 && ffn_pipelined_ok(N, Kd) && kb % kP4BK == 0 && (Kd == kb || Kd == 2 * kb) &&
           (size_t)kb * N * 2 < 0x80000000ull;
}

// C = A [B0^T ; B1^T] per expert, B0 and B1 given as N x kb row-major matrices
// per expert (B1 only when Kd = 2 kb), pipelined kernel only (ffn_bt_ok()).
hipError_t launch_ffn_bt(const void* A, const void* B0, const void* B1, int kb, int dtype, int rows, int N, int E,
                         int Kd, const int32_t* counts, const int32_t* offsets, void* C, float* part,
                         bool tickets_zeroed, hipStream_t s) {
    if (!ffn_bt_ok(dtype, N, Kd, kb) || (Kd == 2 * kb) != (B1 != nullptr)) return hipErrorInvalidValue;
    return launch_pipelined<false, true>(static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B0),
                                         static_cast<const uint16_t*>(B1), static_cast<uint16_t*>(C), counts, offsets,
                                         E, Kd, N, rows, part, tickets_zeroed, nullptr, 1, 1, s, kb);
}

// dA = A B0^T per expert (B0 as for launch_ffn_bt with Kd = kb) with the
// SwiGLU backward fused into the epilogue (BwdEpi): writes dH = [dh1 | dh3],
// w * act (when aw is not null) and the dS parts ds_part [rows, N / 64];
// dA itself is not stored.  Pipelined kernel only (ffn_bt_ok(1, N, kb, kb)).
hipError_t launch_ffn_bt_swiglu_bwd(const void* A, const void* B0, int kb, int rows, int N, int E,
                                    const int32_t* counts, const int32_t* offsets, const void* H1, const void* H3,
                                    void* dH, void* aw, const float* wrow, float* ds_part, hipStream_t s) {
    if (!ffn_bt_ok(1, N, kb, kb)) return hipErrorInvalidValue;
    const BwdEpi ep{static_cast<const uint16_t*>(H1), static_cast<const uint16_t*>(H3), static_cast<uint16_t*>(dH),
                    static_cast<uint16_t*>(aw), wrow, ds_part};
    return launch_pipelined<false, true, true>(static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B0),
                                               nullptr, nullptr, counts, offsets, E, kb, N, rows, nullptr, false,
                                               nullptr, 1, 1, s, kb, ep);
}

hipError_t launch_ffn(const void* Xp, const void* W1, const void* W3, const void* W2, int dtype,
                      int rows, int d, int E, int n, const int32_t* counts, const int32_t* offsets,
                      void* Act, void* Y, float* part, bool tickets_zeroed, hipStream_t s,
                      const int32_t* gather, int gK, int xrows) {
    const hipError_t err = launch_ffn_up(Xp, W1, W3, dtype, rows, d, E, n, counts, offsets, Act, part,
                                         tickets_zeroed, s, gather, gK, xrows);
    if (err != hipSuccess) return err;
    return launch_ffn_down(Act, W2, dtype, rows, d, E, n, counts, offsets, Y, part, tickets_zeroed, s);
}

}  // namespace moe
