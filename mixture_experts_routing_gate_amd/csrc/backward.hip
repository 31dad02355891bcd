// Backward of the MoE layer: dX, the router-logit gradient and (for
// moe_backward) the expert-weight gradients from dout = dL/d(out).  Page [P4] "MoE architecture optimisation and
// SonicMoE practice" section 2.2 names the products the backward needs beside
// the weight gradients: dH through the SwiGLU and dS, the gradient of the
// routing scores, taken as <dA, A> (the activation gradient before the score
// scaling against the activation) so that the expert outputs Y need not be
// kept; section 5 measures the backward.  Per assignment (t, k) with expert e
// and weight w, row p of the expert-sorted order, g = dout[t]:
//   dA  = g W2[e]^T                    (grouped GEMM over the rows)
//   dS  = <dA, SiLU(h1) * h3>          (h1, h3 recomputed by grouped GEMMs)
//   dh1 = w dA h3 SiLU'(h1),  dh3 = w dA SiLU(h1)
//   dXp = [dh1 | dh3] [W1[e]^T ; W3[e]^T]   (grouped GEMM, K = 2n)
//   dX[t] = sum_k dXp[row of (t, k)]   (the combine with unit weights)
//   dlogits[t, idx_k] = w_k (dS_k - sum_j w_j dS_j), 0 for experts not chosen.
// The GEMMs are the forward's grouped kernels (reading the weights as stored,
// k-contiguous, or transposed copies where that mode does not apply); with
// bf16 the SwiGLU backward and dS run in the dA GEMM's epilogue (ffn.hip), and
// this file adds the row weights and the fixed-order dS reduction for it.  It
// also holds the kernels that are new: the weight transpose, the SwiGLU
// backward with dS as its own pass, the logit gradient, a fill, and the weight gradients
//   dW1[e] = Xp^T dh1, dW3[e] = Xp^T dh3, dW2[e] = (w a)^T dY
// summed over each expert's rows (its own kernel: the reduction runs over the
// ragged rows, so tiles are indexed by expert rather than by row).
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kTr = 32;  // fp32 transpose tile
constexpr int kTr16 = 64;  // bf16 transpose tile: rows of 128 bytes

// out[e*oes + c*ors + r] = in[e][r][c] for in [E][R][C]; one 32 x 32 tile per
// workgroup (256 threads), through LDS.  fp32.
template <typename T>
__global__ __launch_bounds__(256) void transpose_experts_kernel(const T* __restrict__ in, int R, int C,
                                                                T* __restrict__ out, size_t oes, size_t ors) {
    __shared__ T tile[kTr][kTr + 1];
    const int tx = threadIdx.x & (kTr - 1), ty = threadIdx.x / kTr;  // ty in 0..7
    const int c0 = blockIdx.x * kTr, r0 = blockIdx.y * kTr;
    const size_t e = blockIdx.z;
    const T* src = in + e * (size_t)R * C;
#pragma unroll
    for (int i = 0; i < kTr / 8; ++i) {
        const int r = r0 + ty + 8 * i, c = c0 + tx;
        if (r < R && c < C) tile[ty + 8 * i][tx] = src[(size_t)r * C + c];
    }
    __syncthreads();
    T* dst = out + e * oes;
#pragma unroll
    for (int i = 0; i < kTr / 8; ++i) {
        const int c = c0 + ty + 8 * i, r = r0 + tx;
        if (r < R && c < C) dst[(size_t)c * ors + r] = tile[tx][ty + 8 * i];
    }
}

// The bf16 transpose, one 64 x 64 tile per workgroup: 16-byte loads along
// the input rows and 16-byte stores along the output rows (8 elements each),
// so that every global access is a whole 128-byte row segment.  R, C, oes and
// ors must be multiples of 8 (whole pieces); tiles past R or C are skipped
// piece by piece.
__global__ __launch_bounds__(256) void transpose_experts_bf16_kernel(const uint16_t* __restrict__ in, int R, int C,
                                                                     uint16_t* __restrict__ out, size_t oes,
                                                                     size_t ors) {
    __shared__ uint16_t tile[kTr16][kTr16 + 2];
    const int c0 = blockIdx.x * kTr16, r0 = blockIdx.y * kTr16;
    const size_t e = blockIdx.z;
    const uint16_t* src = in + e * (size_t)R * C;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int q = threadIdx.x + 256 * h;  // 512 pieces: 64 rows x 8
        const int row = q >> 3, pc = q & 7;
        const int r = r0 + row, c = c0 + pc * 8;
        if (r < R && c < C) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(src + (size_t)r * C + c);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                tile[row][pc * 8 + 2 * i] = (uint16_t)(v[i] & 0xFFFFu);
                tile[row][pc * 8 + 2 * i + 1] = (uint16_t)(v[i] >> 16);
            }
        }
    }
    __syncthreads();
    uint16_t* dst = out + e * oes;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int q = threadIdx.x + 256 * h;  // 64 output rows (c) x 8 pieces of r
        const int col = q >> 3, pr = q & 7;
        const int c = c0 + col, r = r0 + pr * 8;
        if (r < R && c < C) {
            u32x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[i] = (uint32_t)tile[pr * 8 + 2 * i][col] | ((uint32_t)tile[pr * 8 + 2 * i + 1][col] << 16);
            *reinterpret_cast<u32x4*>(dst + (size_t)c * ors + r) = v;
        }
    }
}

MOE_DEV float load_el(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
MOE_DEV float load_el(const float* p, size_t i) { return p[i]; }
MOE_DEV void store_el(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
MOE_DEV void store_el(float* p, size_t i, float v) { p[i] = v; }

// One wave per expert-sorted row p: recomputes a = SiLU(h1) h3 from the
// stored H1, H3 rows, forms dS = <dA, a> (fp32, lane-ordered partial sums,
// then a butterfly: deterministic) and writes dH = [dh1 | dh3] ([rows, 2n]).
// dS goes to dS_tk[sorted_pair[p]] (the (token, slot) order of topk_w).
template <typename T>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const T* __restrict__ H1, const T* __restrict__ H3,
                                                         const T* __restrict__ dA, const float* __restrict__ topk_w,
                                                         const int32_t* __restrict__ sorted_pair, int rows, int n,
                                                         T* __restrict__ dH, float* __restrict__ dS_tk,
                                                         T* __restrict__ aw) {
    const int lane = threadIdx.x & (kWave - 1);
    const int p = blockIdx.x * 4 + threadIdx.x / kWave;
    if (p >= rows) return;
    const int tk = sorted_pair[p];
    const float w = topk_w[tk];
    const size_t rb = (size_t)p * n;
    float ds = 0.0f;
    for (int j = lane; j < n; j += kWave) {
        const float h1 = load_el(H1, rb + j), h3 = load_el(H3, rb + j), g = load_el(dA, rb + j);
        const float sig = 1.0f / (1.0f + expf(-h1));
        const float s1 = h1 * sig;
        ds = fmaf(g, s1 * h3, ds);
        const float wg = w * g;
        store_el(dH, 2 * rb + j, wg * h3 * sig * (1.0f + h1 * (1.0f - sig)));
        store_el(dH, 2 * rb + n + j, wg * s1);
        if (aw != nullptr) store_el(aw, rb + j, w * (s1 * h3));
    }
    ds = group_sum<kWave>(ds);
    if (lane == 0) dS_tk[tk] = ds;
}

// The bf16 SwiGLU backward with 8 elements per lane (16-byte loads and
// stores); n must be a multiple of 8.  Same arithmetic as above per element.
__global__ __launch_bounds__(256) void swiglu_bwd_bf16_kernel(const uint16_t* __restrict__ H1,
                                                              const uint16_t* __restrict__ H3,
                                                              const uint16_t* __restrict__ dA,
                                                              const float* __restrict__ topk_w,
                                                              const int32_t* __restrict__ sorted_pair, int rows, int n,
                                                              uint16_t* __restrict__ dH, float* __restrict__ dS_tk,
                                                              uint16_t* __restrict__ aw) {
    const int lane = threadIdx.x & (kWave - 1);
    const int p = blockIdx.x * 4 + threadIdx.x / kWave;
    if (p >= rows) return;
    const int tk = sorted_pair[p];
    const float w = topk_w[tk];
    const size_t rb = (size_t)p * n;
    float ds = 0.0f;
    for (int j = lane * 8; j < n; j += kWave * 8) {
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(H1 + rb + j);
        const u32x4 a3 = *reinterpret_cast<const u32x4*>(H3 + rb + j);
        const u32x4 ga = *reinterpret_cast<const u32x4*>(dA + rb + j);
        u32x4 o1, o3, oa;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float r1[2], r3[2], ra[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const float h1 = bf16_to_f32((uint16_t)(a1[i] >> (16 * hh)));
                const float h3 = bf16_to_f32((uint16_t)(a3[i] >> (16 * hh)));
                const float g = bf16_to_f32((uint16_t)(ga[i] >> (16 * hh)));
                const float sig = 1.0f / (1.0f + expf(-h1));
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
        *reinterpret_cast<u32x4*>(dH + 2 * rb + j) = o1;
        *reinterpret_cast<u32x4*>(dH + 2 * rb + n + j) = o3;
        if (aw != nullptr) *reinterpret_cast<u32x4*>(aw + rb + j) = oa;
    }
    ds = group_sum<kWave>(ds);
    if (lane == 0) dS_tk[tk] = ds;
}

// wrow[p] = topk_w[sorted_pair[p]]: the routing weight of each expert-sorted row.
__global__ __launch_bounds__(256) void row_weights_kernel(const float* __restrict__ topk_w,
                                                          const int32_t* __restrict__ sorted_pair, int rows,
                                                          float* __restrict__ wrow) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p < rows) wrow[p] = topk_w[sorted_pair[p]];
}

// One wave per row: dS of row p = the sum of its nparts parts, added in part
// order (each lane a strided run, then a butterfly: deterministic), written to
// dS_tk[sorted_pair[p]].
__global__ __launch_bounds__(256) void ds_reduce_kernel(const float* __restrict__ ds_part, int nparts,
                                                        const int32_t* __restrict__ sorted_pair, int rows,
                                                        float* __restrict__ dS_tk) {
    const int lane = threadIdx.x & (kWave - 1);
    const int p = blockIdx.x * 4 + threadIdx.x / kWave;
    if (p >= rows) return;
    const float* src = ds_part + (size_t)p * nparts;
    float ds = 0.0f;
    for (int j = lane; j < nparts; j += kWave) ds += src[j];
    ds = group_sum<kWave>(ds);
    if (lane == 0) dS_tk[sorted_pair[p]] = ds;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, lane i gets element i%4 of the
// 8-byte pieces addressed by lanes i/4, 4+i/4, 8+i/4 and 12+i/4 (a 4 x 16 ->
// 16 x 4 transpose of 16-bit values).
MOE_DEV bf16x4 lds_tr4(const char* l) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(l)));
}

// Weight gradient of one expert's linear map, summed over its rows:
//   dW[e][m][c] = sum over rows r of expert e of P[r][m] * Q[r][qoff + c]
// (fp32 out, [E, M, N]).  For dW1 / dW3: P = the expert-sorted X, Q = the
// dh1 / dh3 halves of dH; for dW2: P = w * act, Q = the expert-sorted dout.
// One 128 x 128 tile of one expert per workgroup, four waves of 64 x 64 on
// v_mfma_f32_32x32x16_bf16; the rows are the reduction, 64 at a time.  Both
// operands arrive row-major (the reduction index outermost), so each 64-row
// slab is stored as it is read, in 16-byte pieces (row r at r * 256 bytes,
// piece c at position c ^ 4*(r % 4)), and the MFMA fragments (8 consecutive
// rows per lane) come from transposing LDS reads.  Rows past the expert's
// count read as zeros.  The sum runs over rows in ascending order.
__global__ __launch_bounds__(256, 2) void dw_bf16_kernel(const uint16_t* __restrict__ P, int ldp,
                                                         const uint16_t* __restrict__ Q, int ldq, int qoff,
                                                         const int32_t* __restrict__ counts,
                                                         const int32_t* __restrict__ offsets, int M, int N, int rows,
                                                         float* __restrict__ dW) {
    constexpr int BM = 128, BN = 128, BK = 64, SLAB = BK * 256;  // 16 KB per operand
    __shared__ __attribute__((aligned(1024))) char Ps[SLAB];
    __shared__ __attribute__((aligned(1024))) char Qs[SLAB];
    const int MT = M / BM, NT = N / BN;
    const int tile = blockIdx.x;
    const int e = tile / (MT * NT), rem = tile % (MT * NT);
    const int m0 = (rem / NT) * BM, n0 = (rem % NT) * BN;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const int g16 = lane >> 4, s16 = lane & 15;
    const int cnt = counts[e];
    const int r0 = offsets[e];
    // rows of the expert that exist; never past the end of P/Q whatever counts/offsets hold
    const int nr = (r0 < 0 || r0 >= rows || cnt <= 0) ? 0 : min(cnt, rows - r0);
    // byte offset of this lane's transposing read for the 32-column block starting at column cb
    const int rd_lane = ((g16 >> 1) * 8 + (s16 >> 2)) * 256 + (s16 & 1) * 8;
    const int rd_x = (s16 >> 2) << 2, rd_c = (g16 & 1) * 2 + ((s16 & 3) >> 1);
    auto rd = [&](int cb) { return rd_lane + ((((cb >> 3) ^ rd_x) + rd_c) << 4); };
    int pa[2], qa[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        pa[i] = rd(wm * 64 + i * 32);
        qa[i] = rd(wn * 64 + i * 32);
    }

    f32x16 acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.0f;

    for (int k0 = 0; k0 < nr; k0 += BK) {
        __syncthreads();
        // BK rows x 16 pieces of 8 columns per operand: all loads issued, then all stores
        u32x4 vp[BK / 16], vq[BK / 16];
#pragma unroll
        for (int i = 0; i < BK / 16; ++i) {
            const int c = tid + 256 * i;
            const int kr = c >> 4, pc = c & 15;
            vp[i] = u32x4{0u, 0u, 0u, 0u};
            vq[i] = u32x4{0u, 0u, 0u, 0u};
            if (k0 + kr < nr) {
                const size_t r = (size_t)(r0 + k0 + kr);
                vp[i] = *reinterpret_cast<const u32x4*>(P + r * ldp + m0 + pc * 8);
                vq[i] = *reinterpret_cast<const u32x4*>(Q + r * ldq + qoff + n0 + pc * 8);
            }
        }
#pragma unroll
        for (int i = 0; i < BK / 16; ++i) {
            const int c = tid + 256 * i;
            const int kr = c >> 4, pc = c & 15;
            const int off = kr * 256 + ((pc ^ ((kr & 3) << 2)) << 4);
            *reinterpret_cast<u32x4*>(Ps + off) = vp[i];
            *reinterpret_cast<u32x4*>(Qs + off) = vq[i];
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const char* pp = Ps + pa[i] + ks * 16 * 256;
                const char* qq = Qs + qa[i] + ks * 16 * 256;
                a[i] = __builtin_shufflevector(lds_tr4(pp), lds_tr4(pp + 4 * 256), 0, 1, 2, 3, 4, 5, 6, 7);
                b[i] = __builtin_shufflevector(lds_tr4(qq), lds_tr4(qq + 4 * 256), 0, 1, 2, 3, 4, 5, 6, 7);
            }
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
        }
    }
    // element i of lane l: row (i/4)*8 + (l/32)*4 + i%4, column l%32 of the 32 x 32 block
    float* out = dW + (size_t)e * M * N;
    const int l32 = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = m0 + wm * 64 + mi * 32 + (i >> 2) * 8 + lh * 4 + (i & 3);
                const int col = n0 + wn * 64 + ni * 32 + l32;
                out[(size_t)row * N + col] = acc[mi][ni][i];
            }
}

// The same sum in fp32: one thread per output element, rows in ascending order.
__global__ __launch_bounds__(256) void dw_f32_kernel(const float* __restrict__ P, int ldp, const float* __restrict__ Q,
                                                     int ldq, int qoff, const int32_t* __restrict__ counts,
                                                     const int32_t* __restrict__ offsets, int E, int M, int N,
                                                     int rows, float* __restrict__ dW) {
    const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= (size_t)E * M * N) return;
    const int e = (int)(q / ((size_t)M * N));
    const size_t rem = q % ((size_t)M * N);
    const int m = (int)(rem / N), c = (int)(rem % N);
    const int cnt = counts[e], r0 = offsets[e];
    const int nr = (r0 < 0 || r0 >= rows || cnt <= 0) ? 0 : min(cnt, rows - r0);
    float acc = 0.0f;
    for (int k = 0; k < nr; ++k) {
        const size_t r = (size_t)(r0 + k);
        acc = fmaf(P[r * ldp + m], Q[r * ldq + qoff + c], acc);
    }
    dW[q] = acc;
}

// dlogits[t, e] = w_k (dS_k - sum_j w_j dS_j) when e = idx[t, k], else 0;
// one thread per (t, e).
__global__ __launch_bounds__(256) void logit_grad_kernel(const int32_t* __restrict__ idx,
                                                         const float* __restrict__ topk_w,
                                                         const float* __restrict__ dS_tk, int T, int E, int K,
                                                         float* __restrict__ dlogits) {
    const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= (size_t)T * E) return;
    const size_t t = q / E;
    const int e = (int)(q % E);
    float mean = 0.0f;
    for (int k = 0; k < K; ++k) mean = fmaf(topk_w[t * K + k], dS_tk[t * K + k], mean);
    float g = 0.0f;
    for (int k = 0; k < K; ++k)
        if (idx[t * K + k] == e) g = topk_w[t * K + k] * (dS_tk[t * K + k] - mean);
    dlogits[q] = g;
}

__global__ __launch_bounds__(256) void fill_f32_kernel(float* __restrict__ p, size_t n, float v) {
    for (size_t q = (size_t)blockIdx.x * 256 + threadIdx.x; q < n; q += (size_t)gridDim.x * 256) p[q] = v;
}

}  // namespace

hipError_t launch_transpose_experts(const void* in, int dtype, int E, int R, int C, void* out, size_t oes,
                                    size_t ors, hipStream_t s) {
    const dim3 grid((unsigned)((C + kTr - 1) / kTr), (unsigned)((R + kTr - 1) / kTr), (unsigned)E);
    if (dtype == 1) {
        const dim3 g16((unsigned)((C + kTr16 - 1) / kTr16), (unsigned)((R + kTr16 - 1) / kTr16), (unsigned)E);
        hipLaunchKernelGGL(transpose_experts_bf16_kernel, g16, dim3(256), 0, s, static_cast<const uint16_t*>(in), R,
                           C, static_cast<uint16_t*>(out), oes, ors);
    } else
        hipLaunchKernelGGL(transpose_experts_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(in),
                           R, C, static_cast<float*>(out), oes, ors);
    return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const void* H1, const void* H3, const void* dA, const float* topk_w,
                             const int32_t* sorted_pair, int dtype, int rows, int n, void* dH, float* dS_tk,
                             void* aw, hipStream_t s) {
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (rows <= 0) return hipSuccess;
    if (dtype == 1)
        hipLaunchKernelGGL(swiglu_bwd_bf16_kernel, grid, dim3(256), 0, s, static_cast<const uint16_t*>(H1),
                           static_cast<const uint16_t*>(H3), static_cast<const uint16_t*>(dA), topk_w, sorted_pair,
                           rows, n, static_cast<uint16_t*>(dH), dS_tk, static_cast<uint16_t*>(aw));
    else
        hipLaunchKernelGGL(swiglu_bwd_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(H1),
                           static_cast<const float*>(H3), static_cast<const float*>(dA), topk_w, sorted_pair, rows,
                           n, static_cast<float*>(dH), dS_tk, static_cast<float*>(aw));
    return hipGetLastError();
}

hipError_t launch_dw(const void* P, int ldp, const void* Q, int ldq, int qoff, const int32_t* counts,
                     const int32_t* offsets, int dtype, int E, int M, int N, int rows, float* dW, hipStream_t s) {
    if (dw_p4_ok(dtype, E, M, N, rows, ldp, ldq))
        return launch_dw_p4(P, ldp, Q, ldq, qoff, counts, offsets, E, M, N, rows, dW, s);
    if (dtype == 1) {
        const unsigned tiles = (unsigned)((size_t)E * (M / 128) * (N / 128));
        hipLaunchKernelGGL(dw_bf16_kernel, dim3(tiles), dim3(256), 0, s, static_cast<const uint16_t*>(P), ldp,
                           static_cast<const uint16_t*>(Q), ldq, qoff, counts, offsets, M, N, rows, dW);
    } else {
        const size_t nel = (size_t)E * M * N;
        hipLaunchKernelGGL(dw_f32_kernel, dim3((unsigned)((nel + 255) / 256)), dim3(256), 0, s,
                           static_cast<const float*>(P), ldp, static_cast<const float*>(Q), ldq, qoff, counts,
                           offsets, E, M, N, rows, dW);
    }
    return hipGetLastError();
}

hipError_t launch_row_weights(const float* topk_w, const int32_t* sorted_pair, int rows, float* wrow, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(row_weights_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, topk_w, sorted_pair,
                       rows, wrow);
    return hipGetLastError();
}

hipError_t launch_ds_reduce(const float* ds_part, int nparts, const int32_t* sorted_pair, int rows, float* dS_tk,
                            hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(ds_reduce_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, ds_part, nparts,
                       sorted_pair, rows, dS_tk);
    return hipGetLastError();
}

hipError_t launch_logit_grad(const int32_t* idx, const float* topk_w, const float* dS_tk, int T, int E, int K,
                             float* dlogits, hipStream_t s) {
    const size_t n = (size_t)T * E;
    hipLaunchKernelGGL(logit_grad_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, idx, topk_w, dS_tk, T,
                       E, K, dlogits);
    return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, size_t n, float v, hipStream_t s) {
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

}  // namespace moe
