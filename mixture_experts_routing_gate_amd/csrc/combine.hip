// Step 5 of the MoE layer forward: gate-weighted combine back to token order.
//
// Page [P4] "MoE architecture optimisation and SonicMoE practice" section 1
// (scatter: results go back to their token positions) and page [P2] "SpMM in
// MoE" sections 1 and 6 (the selected experts' outputs are averaged with the
// gate weights).  Written as a gather-sum by token so that no two lanes ever
// add into the same output: out[t] = sum_k w[t,k] * Y[inv[t*K+k]], k in order,
// fp32 fused multiply-adds, rounded once to the storage type.  No atomics, so
// the result is bitwise reproducible.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// One wave per token; each lane owns 16-byte chunks of the row (8 bf16 or 4 fp32).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void combine_kernel(const u32x4* __restrict__ Y,
                                                           const float* __restrict__ w,
                                                           const int32_t* __restrict__ inv, int T,
                                                           int row_chunks, int K,
                                                           u32x4* __restrict__ out) {
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * kWaves + threadIdx.x / kWave;
    if (t >= T) return;
    const int A = T * K;
    int pos[8];
    float wk[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        pos[k] = -1;
        wk[k] = 0.0f;
        if (k < K) {
            pos[k] = uniform(inv[(size_t)t * K + k]);
            if ((unsigned)pos[k] >= (unsigned)A) pos[k] = -1;  // never read outside Y, whatever inv holds
            wk[k] = __builtin_bit_cast(float, uniform(__builtin_bit_cast(int, w[(size_t)t * K + k])));
        }
    }
    for (int c = lane; c < row_chunks; c += kWave) {
        u32x4 y[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (k < K && pos[k] >= 0) y[k] = __builtin_nontemporal_load(Y + (size_t)pos[k] * row_chunks + c);
        constexpr int NV = BF16 ? 8 : 4;
        float acc[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) acc[i] = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (k < K && pos[k] >= 0) {
#pragma unroll
                for (int i = 0; i < NV; ++i) {
                    float yi;
                    if (BF16)
                        yi = bf16_to_f32((uint16_t)(y[k][i / 2] >> (16 * (i & 1))));
                    else
                        yi = __uint_as_float(y[k][i]);
                    acc[i] = fmaf(wk[k], yi, acc[i]);
                }
            }
        }
        u32x4 o;
        if (BF16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(acc[i]);
        }
        out[(size_t)t * row_chunks + c] = o;
    }
}

}  // namespace

hipError_t launch_combine(const void* Y, const float* w, const int32_t* inv, int dtype, int T, int d,
                          int K, void* out, hipStream_t s) {
    const size_t row_bytes = (size_t)d * (dtype == 1 ? 2 : 4);
    const int row_chunks = (int)(row_bytes / 16);
    const dim3 grid((T + kWaves - 1) / kWaves);
    if (dtype == 1)
        hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(kThreads), 0, s,
                           static_cast<const u32x4*>(Y), w, inv, T, row_chunks, K,
                           static_cast<u32x4*>(out));
    else
        hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(kThreads), 0, s,
                           static_cast<const u32x4*>(Y), w, inv, T, row_chunks, K,
                           static_cast<u32x4*>(out));
    return hipGetLastError();
}

}  // namespace moe
