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
// K <= KC; each lane keeps U * KC row loads in flight (U chunks of each of the
// K source rows) before the first multiply-add: 4 for K = 2, 8 for K = 1 and
// K <= 4, 16 for K <= 8 (measured best on the Mixtral-, fine- and
// DeepSeek-V3-shaped layers).  The
// output row is written with streaming stores: it is not read again here.
template <bool BF16, int KC>
__global__ __launch_bounds__(kThreads) void combine_kernel(const u32x4* __restrict__ Y,
                                                           const float* __restrict__ w,
                                                           const int32_t* __restrict__ inv, int T,
                                                           int row_chunks, int K,
                                                           u32x4* __restrict__ out) {
    constexpr int U = KC == 8 ? 2 : KC == 2 ? 2 : 8 / KC;
    constexpr int NV = BF16 ? 8 : 4;
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * kWaves + threadIdx.x / kWave;
    if (t >= T) return;
    const int A = T * K;
    int pos[KC];
    float wk[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        pos[k] = -1;
        wk[k] = 0.0f;
        if (k < K) {
            pos[k] = uniform(inv[(size_t)t * K + k]);
            if ((unsigned)pos[k] >= (unsigned)A) pos[k] = -1;  // never read outside Y, whatever inv holds
            wk[k] = __builtin_bit_cast(float, uniform(__builtin_bit_cast(int, w[(size_t)t * K + k])));
        }
    }
    u32x4* orow = out + (size_t)t * row_chunks;
    for (int c0 = 0; c0 < row_chunks; c0 += kWave * U) {
        u32x4 y[U][KC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * kWave + lane;
#pragma unroll
            for (int k = 0; k < KC; ++k)
                if (c < row_chunks && k < K && pos[k] >= 0)
                    y[u][k] = __builtin_nontemporal_load(Y + (size_t)pos[k] * row_chunks + c);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * kWave + lane;
            if (c >= row_chunks) break;
            float acc[NV];
#pragma unroll
            for (int i = 0; i < NV; ++i) acc[i] = 0.0f;
#pragma unroll
            for (int k = 0; k < KC; ++k) {
                if (k < K && pos[k] >= 0) {
#pragma unroll
                    for (int i = 0; i < NV; ++i) {
                        float yi;
                        if (BF16)
                            yi = bf16_to_f32((uint16_t)(y[u][k][i / 2] >> (16 * (i & 1))));
                        else
                            yi = __uint_as_float(y[u][k][i]);
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
            __builtin_nontemporal_store(o, orow + c);
        }
    }
}

template <bool BF16, int KC>
void launch_combine_k(const void* Y, const float* w, const int32_t* inv, int T, int row_chunks, int K,
                      void* out, hipStream_t s) {
    hipLaunchKernelGGL((combine_kernel<BF16, KC>), dim3((T + kWaves - 1) / kWaves), dim3(kThreads), 0, s,
                       static_cast<const u32x4*>(Y), w, inv, T, row_chunks, K, static_cast<u32x4*>(out));
}

template <bool BF16>
void launch_combine_t(const void* Y, const float* w, const int32_t* inv, int T, int row_chunks, int K,
                      void* out, hipStream_t s) {
    if (K <= 1) launch_combine_k<BF16, 1>(Y, w, inv, T, row_chunks, K, out, s);
    else if (K <= 2) launch_combine_k<BF16, 2>(Y, w, inv, T, row_chunks, K, out, s);
    else if (K <= 4) launch_combine_k<BF16, 4>(Y, w, inv, T, row_chunks, K, out, s);
    else launch_combine_k<BF16, 8>(Y, w, inv, T, row_chunks, K, out, s);
}

}  // namespace

hipError_t launch_combine(const void* Y, const float* w, const int32_t* inv, int dtype, int T, int d,
                          int K, void* out, hipStream_t s) {
    const size_t row_bytes = (size_t)d * (dtype == 1 ? 2 : 4);
    const int row_chunks = (int)(row_bytes / 16);
    if (dtype == 1) launch_combine_t<true>(Y, w, inv, T, row_chunks, K, out, s);
    else launch_combine_t<false>(Y, w, inv, T, row_chunks, K, out, s);
    return hipGetLastError();
}

}  // namespace moe
