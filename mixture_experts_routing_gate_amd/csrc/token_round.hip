// Token Rounding: the routing variant of page [P4] "MoE architecture
// optimisation and SonicMoE practice", section 3.  The per-expert counts of
// ordinary top-K routing are rounded to whole tiles of M rows (section 3.1),
// to the nearest multiple with a half rounding up (the rounding of section
// 3.2), at most cap_tiles tiles per expert when a limit is given (section
// 3.2 names 2M tokens), and never above T.  A second sort by score decides
// which tokens each expert drops or takes on: ranked by logit descending, then
// token ascending, an expert rounded down keeps its best routed tokens and an
// expert rounded up keeps all of them plus the best tokens not routed to it.
// Each token's weights are then a softmax over the experts it kept (the
// renormalisation of section 3.2).
//
// Layout of the plan: rows expert by expert, tokens ascending inside an
// expert (row_tok[row] = token), and per (token, expert) the row it occupies
// or -1 (slot_row[T,E]) and its weight or 0 (slot_w[T,E]).
//
// Kernels, in stream order:
//   tr_keys_kernel     logits [T,E] and topk_idx -> per expert, over tokens:
//                      the logit's order key and a routed flag ([E,T], LDS
//                      tile transpose);
//   tr_select_kernel   one workgroup per expert: its target row count, its
//                      row offset, a 4-pass radix select of the m-th best
//                      candidate key, then the kept tokens in ascending order;
//   tr_slots_kernel    per token: slot_row and the softmax over kept experts;
//   tr_combine_kernel  per token: sum over kept experts, ascending, of
//                      slot_w * Y[slot_row], fp32, rounded once;
//   tr_gather_rows_kernel  X rows in plan order, for the grouped GEMMs that
//                      do not gather on load.
// Every decision compares fp32 logits exactly, and the selection and layout
// use integer counts only, so the plan is reproducible bit for bit.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

// Order key of an fp32 value: unsigned comparison of keys orders the values
// (x + 0.0f folds -0.0 into +0.0, so the two compare equal, as floats do).
MOE_DEV uint32_t tr_ord_key(float x) {
    const uint32_t u = __float_as_uint(x + 0.0f);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Rows an expert with f routed tokens keeps (same rule on host and device).
MOE_DEV int tr_target_dev(int f, int M, int T, int cap_tiles) {
    long long r = (((long long)f + M / 2) / M) * M;
    if (r > T) r -= M;
    if (cap_tiles > 0 && r > (long long)cap_tiles * M) r = (long long)cap_tiles * M;
    return (int)r;
}

constexpr int kTile = 32;  // tokens x experts per transpose tile

// keyT[e*T + t] = order key of logits[t,e]; memT[e*T + t] = 1 when e is one
// of topk_idx[t, 0..K) (entries outside [0,E) are ignored), else 0.
__global__ __launch_bounds__(256) void tr_keys_kernel(const float* __restrict__ logits,
                                                      const int32_t* __restrict__ idx, int T, int E, int K,
                                                      uint32_t* __restrict__ keyT, uint8_t* __restrict__ memT) {
    __shared__ uint32_t s_key[kTile][kTile + 1];
    __shared__ uint8_t s_mem[kTile][kTile + 1];
    const int tx = threadIdx.x & (kTile - 1), ty = threadIdx.x / kTile;  // ty in 0..7
    const int t0 = blockIdx.x * kTile, e0 = blockIdx.y * kTile;
#pragma unroll
    for (int i = 0; i < kTile / 8; ++i) {
        const int tt = ty + 8 * i;
        const int t = t0 + tt, e = e0 + tx;
        s_mem[tt][tx] = 0;
        if (t < T && e < E) s_key[tt][tx] = tr_ord_key(logits[(size_t)t * E + e]);
    }
    __syncthreads();
    for (int q = threadIdx.x; q < kTile * K; q += 256) {
        const int tt = q / K;
        const int t = t0 + tt;
        if (t < T) {
            const int ex = idx[(size_t)t * K + q % K];
            if (ex >= e0 && ex < e0 + kTile && ex < E) s_mem[tt][ex - e0] = 1;
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kTile / 8; ++i) {
        const int ee = ty + 8 * i;
        const int e = e0 + ee, t = t0 + tx;
        if (t < T && e < E) {
            keyT[(size_t)e * T + t] = s_key[tx][ee];
            memT[(size_t)e * T + t] = s_mem[tx][ee];
        }
    }
}

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;

// Exclusive prefix count of `flag` over the workgroup in thread order; *total
// gets the workgroup's count.  Every thread must call it.
MOE_DEV int block_excl_count(bool flag, int* s_wave, int* total) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const unsigned long long b = __ballot(flag);
    const int in_wave = __popcll(b & ((1ull << lane) - 1ull));
    if (lane == 0) s_wave[wave] = __popcll(b);
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        const int v = s_wave[w];
        before += w < wave ? v : 0;
        tot += v;
    }
    __syncthreads();
    *total = tot;
    return before + in_wave;
}

// Workgroup sum of a 64-bit value (fixed order: deterministic).
MOE_DEV long long block_sum_ll(long long v, long long* s_ll) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
    for (int s = 1; s < kWave; s <<= 1) v += __shfl_xor(v, s, kWave);
    if (lane == 0) s_ll[wave] = v;
    __syncthreads();
    long long tot = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) tot += s_ll[w];
    __syncthreads();
    return tot;
}

// One workgroup per expert e.  counts[] is the histogram of topk_idx (as
// moe_route writes it); rows of e are [o, o + r) with o the sum of the targets
// of the experts before e.  Writes counts_r[e], offsets_r[e] (and offsets_r[E]
// from the last expert), row_tok[o .. o+r) and slotT[e*T + t] for every t.
// Nothing is written past rows_cap rows, whatever counts holds.
__global__ __launch_bounds__(kSelThreads) void tr_select_kernel(
    const uint32_t* __restrict__ keyT, const uint8_t* __restrict__ memT, int T, int E, int M, int cap_tiles,
    const int32_t* __restrict__ counts, int32_t* __restrict__ counts_r, int32_t* __restrict__ offsets_r,
    int32_t* __restrict__ row_tok, long long rows_cap, int32_t* __restrict__ slotT) {
    __shared__ int s_hist[256];
    __shared__ int s_wave[kSelWaves];
    __shared__ long long s_ll[kSelWaves];
    __shared__ int s_digit, s_above, s_total;
    const int tid = threadIdx.x;
    const int e = blockIdx.x;
    const uint32_t* key = keyT + (size_t)e * T;
    const uint8_t* mem = memT + (size_t)e * T;
    int32_t* srow = slotT + (size_t)e * T;

    long long part = 0;
    for (int q = tid; q < e; q += kSelThreads) part += tr_target_dev(min(max(counts[q], 0), T), M, T, cap_tiles);
    const long long o = block_sum_ll(part, s_ll);
    const int f = min(max(counts[e], 0), T);
    const int r = tr_target_dev(f, M, T, cap_tiles);
    const bool room = o + r <= rows_cap;
    if (tid == 0) {
        counts_r[e] = r;
        offsets_r[e] = (int32_t)o;
        if (e == E - 1) offsets_r[E] = (int32_t)(o + r);
    }

    // Rounded down: candidates are the routed tokens, keep the best r.
    // Rounded up: every routed token stays; candidates are the others, take the best r - f.
    const bool down = r <= f;
    const uint8_t want = down ? 1 : 0;
    const int m = down ? r : r - f;

    // Radix select, 8 bits a pass from the top: tau = key of the m-th best
    // candidate, need = how many candidates equal to tau are taken (the lowest
    // tokens).  take_all when there are no more than m candidates.
    uint32_t tau = 0;
    int need = 0;
    bool take_all = false;
    if (m > 0) {
        uint32_t prefix = 0, hmask = 0;
        need = m;
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            if (tid < 256) s_hist[tid] = 0;
            __syncthreads();
            for (int t = tid; t < T; t += kSelThreads) {
                if (mem[t] == want) {
                    const uint32_t k = key[t];
                    if ((k & hmask) == prefix) atomicAdd(&s_hist[(k >> shift) & 255u], 1);
                }
            }
            __syncthreads();
            // above(b) = candidates in bins above b: a suffix sum, one bin per thread
            if (tid < 256) {
                int above = 0;
                for (int b = 255; b > tid; --b) above += s_hist[b];
                const int v = s_hist[tid];
                if (above < need && need <= above + v) {
                    s_digit = tid;
                    s_above = above;
                }
                if (tid == 0) s_total = above + v;
            }
            __syncthreads();
            if (pass == 0 && s_total <= need) {
                take_all = true;
                break;
            }
            prefix |= (uint32_t)s_digit << shift;
            hmask |= 0xFFu << shift;
            need -= s_above;
            __syncthreads();
        }
        tau = prefix;
    }

    // Kept tokens in ascending order.
    int base_sel = 0, base_tie = 0;
    for (int t0 = 0; t0 < T; t0 += kSelThreads) {
        const int t = t0 + tid;
        const bool valid = t < T;
        const uint8_t mb = valid ? mem[t] : 0;
        const uint32_t k = valid ? key[t] : 0u;
        const bool cand = valid && m > 0 && mb == want;
        const bool always = valid && !down && mb == 1;
        const bool tie = cand && !take_all && k == tau;
        int tie_total;
        const int tie_rank = base_tie + block_excl_count(tie, s_wave, &tie_total);
        const bool sel = always || (cand && (take_all || k > tau)) || (tie && tie_rank < need);
        int sel_total;
        const int pos = base_sel + block_excl_count(sel, s_wave, &sel_total);
        if (valid) {
            int32_t row = -1;
            if (sel && room && pos < r) {
                row = (int32_t)(o + pos);
                row_tok[row] = t;
            }
            srow[t] = row;
        }
        base_sel += sel_total;
        base_tie += tie_total;
    }
}

constexpr int kSlotTokens = 32;  // tokens per workgroup of tr_slots_kernel

// slot_row[t,e] from slotT[e,t] (through LDS), and slot_w[t,e] = softmax of
// logits[t,:] over the kept experts: exp(l - m) / sum, m the largest kept
// logit, fp32; 0 where not kept.  One wave per token.
__global__ __launch_bounds__(256) void tr_slots_kernel(const float* __restrict__ logits,
                                                       const int32_t* __restrict__ slotT, int T, int E,
                                                       int32_t* __restrict__ slot_row, float* __restrict__ slot_w) {
    extern __shared__ int32_t s_rows[];  // [kSlotTokens][E + 1]
    const int t0 = blockIdx.x * kSlotTokens;
    const int ld = E + 1;
    for (int q = threadIdx.x; q < kSlotTokens * E; q += 256) {
        const int e = q / kSlotTokens, tt = q % kSlotTokens;
        const int t = t0 + tt;
        s_rows[tt * ld + e] = t < T ? slotT[(size_t)e * T + t] : -1;
    }
    __syncthreads();
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    for (int tt = wave; tt < kSlotTokens; tt += 4) {
        const int t = t0 + tt;
        if (t >= T) break;
        const float* l = logits + (size_t)t * E;
        float mx = -INFINITY;
        for (int e = lane; e < E; e += kWave)
            if (s_rows[tt * ld + e] >= 0) mx = fmaxf(mx, l[e]);
        mx = group_max<kWave>(mx);
        float sum = 0.0f;
        for (int e = lane; e < E; e += kWave)
            if (s_rows[tt * ld + e] >= 0) sum += expf(l[e] - mx);
        sum = group_sum<kWave>(sum);
        for (int e = lane; e < E; e += kWave) {
            const int32_t row = s_rows[tt * ld + e];
            slot_row[(size_t)t * E + e] = row;
            slot_w[(size_t)t * E + e] = row >= 0 ? expf(l[e] - mx) / sum : 0.0f;
        }
    }
}

constexpr int kCombineWaves = 4;

// One wave per token.  The kept (row, weight) pairs are listed in ascending
// expert order in LDS; each lane then owns 16-byte chunks of the output row
// and keeps G rows x U chunks of loads in flight before its multiply-adds.
// Rows outside [0, nrows) are skipped.
template <bool BF16>
__global__ __launch_bounds__(kCombineWaves * kWave) void tr_combine_kernel(
    const u32x4* __restrict__ Y, const int32_t* __restrict__ slot_row, const float* __restrict__ slot_w, int T,
    int E, long long nrows, int row_chunks, u32x4* __restrict__ out) {
    constexpr int U = 2, G = 4;
    constexpr int NV = BF16 ? 8 : 4;
    extern __shared__ int32_t s_list[];  // per wave: E rows, then E weights
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int t = blockIdx.x * kCombineWaves + wave;
    const bool active = t < T;
    int32_t* lrow = s_list + wave * 2 * E;
    float* lw = reinterpret_cast<float*>(lrow + E);
    int n = 0;
    for (int e0 = 0; e0 < E; e0 += kWave) {
        const int e = e0 + lane;
        int32_t row = -1;
        float w = 0.0f;
        if (active && e < E) {
            row = slot_row[(size_t)t * E + e];
            w = slot_w[(size_t)t * E + e];
        }
        const bool ok = row >= 0 && (long long)row < nrows;
        const unsigned long long b = __ballot(ok);
        if (ok) {
            const int p = n + __popcll(b & ((1ull << lane) - 1ull));
            lrow[p] = row;
            lw[p] = w;
        }
        n += __popcll(b);
    }
    __syncthreads();
    if (!active) return;
    u32x4* orow = out + (size_t)t * row_chunks;
    for (int c0 = 0; c0 < row_chunks; c0 += kWave * U) {
        float acc[U][NV];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < NV; ++i) acc[u][i] = 0.0f;
        for (int j0 = 0; j0 < n; j0 += G) {
            u32x4 y[G][U];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (j0 + g < n) {
                    const u32x4* src = Y + (size_t)lrow[j0 + g] * row_chunks;
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int c = c0 + u * kWave + lane;
                        if (c < row_chunks) y[g][u] = __builtin_nontemporal_load(src + c);
                    }
                }
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (j0 + g < n) {
                    const float w = lw[j0 + g];
#pragma unroll
                    for (int u = 0; u < U; ++u)
#pragma unroll
                        for (int i = 0; i < NV; ++i) {
                            float yi;
                            if (BF16)
                                yi = bf16_to_f32((uint16_t)(y[g][u][i / 2] >> (16 * (i & 1))));
                            else
                                yi = __uint_as_float(y[g][u][i]);
                            acc[u][i] = fmaf(w, yi, acc[u][i]);
                        }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * kWave + lane;
            if (c >= row_chunks) break;
            u32x4 o;
            if (BF16) {
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[u][2 * i], acc[u][2 * i + 1]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(acc[u][i]);
            }
            __builtin_nontemporal_store(o, orow + c);
        }
    }
}

// Xp[p] = X[row_tok[p]] for the rows of the plan (p < offsets_r[E], at most
// rows_cap); one wave per row, token indices clamped into [0, T).
__global__ __launch_bounds__(256) void tr_gather_rows_kernel(const u32x4* __restrict__ X, int row_chunks, int T,
                                                             const int32_t* __restrict__ row_tok,
                                                             const int32_t* __restrict__ offsets_r, int E,
                                                             long long rows_cap, u32x4* __restrict__ Xp) {
    const long long p = (long long)blockIdx.x * 4 + threadIdx.x / kWave;
    const long long nrows = min((long long)max(offsets_r[E], 0), rows_cap);
    if (p >= nrows) return;
    const int t = min(max(row_tok[p], 0), T - 1);
    const u32x4* src = X + (size_t)t * row_chunks;
    u32x4* dst = Xp + (size_t)p * row_chunks;
    for (int c = threadIdx.x & (kWave - 1); c < row_chunks; c += kWave) dst[c] = src[c];
}

}  // namespace

long long tr_target(int f, int M, int T, int cap_tiles) {
    long long r = (((long long)f + M / 2) / M) * M;
    if (r > T) r -= M;
    if (cap_tiles > 0 && r > (long long)cap_tiles * M) r = (long long)cap_tiles * M;
    return r;
}

size_t tr_keys_bytes(int T, int E) { return (size_t)T * E * (sizeof(uint32_t) + sizeof(uint8_t) + sizeof(int32_t)); }

hipError_t launch_token_round(const float* logits, const int32_t* idx, const int32_t* counts, int T, int E, int K,
                              int M, int cap_tiles, int32_t* counts_r, int32_t* offsets_r, int32_t* row_tok,
                              long long rows_cap, int32_t* slot_row, float* slot_w, void* ws, hipStream_t s) {
    uint32_t* keyT = static_cast<uint32_t*>(ws);
    int32_t* slotT = reinterpret_cast<int32_t*>(keyT + (size_t)T * E);
    uint8_t* memT = reinterpret_cast<uint8_t*>(slotT + (size_t)T * E);
    const dim3 kgrid((unsigned)((T + kTile - 1) / kTile), (unsigned)((E + kTile - 1) / kTile));
    hipLaunchKernelGGL(tr_keys_kernel, kgrid, dim3(256), 0, s, logits, idx, T, E, K, keyT, memT);
    hipLaunchKernelGGL(tr_select_kernel, dim3((unsigned)E), dim3(kSelThreads), 0, s, keyT, memT, T, E, M,
                       cap_tiles, counts, counts_r, offsets_r, row_tok, rows_cap, slotT);
    const size_t lds = (size_t)kSlotTokens * (E + 1) * sizeof(int32_t);
    hipLaunchKernelGGL(tr_slots_kernel, dim3((unsigned)((T + kSlotTokens - 1) / kSlotTokens)), dim3(256), lds, s,
                       logits, slotT, T, E, slot_row, slot_w);
    return hipGetLastError();
}

hipError_t launch_tr_combine(const void* Y, const int32_t* slot_row, const float* slot_w, int dtype, int T, int E,
                             int d, long long nrows, void* out, hipStream_t s) {
    const int row_chunks = (int)((size_t)d * (dtype == 1 ? 2 : 4) / 16);
    const dim3 grid((unsigned)((T + kCombineWaves - 1) / kCombineWaves));
    const size_t lds = (size_t)kCombineWaves * 2 * E * sizeof(int32_t);
    if (dtype == 1)
        hipLaunchKernelGGL(tr_combine_kernel<true>, grid, dim3(kCombineWaves * kWave), lds, s,
                           static_cast<const u32x4*>(Y), slot_row, slot_w, T, E, nrows, row_chunks,
                           static_cast<u32x4*>(out));
    else
        hipLaunchKernelGGL(tr_combine_kernel<false>, grid, dim3(kCombineWaves * kWave), lds, s,
                           static_cast<const u32x4*>(Y), slot_row, slot_w, T, E, nrows, row_chunks,
                           static_cast<u32x4*>(out));
    return hipGetLastError();
}

hipError_t launch_tr_gather_rows(const void* X, size_t row_bytes, int T, const int32_t* row_tok,
                                 const int32_t* offsets_r, int E, long long rows_cap, void* Xp, hipStream_t s) {
    const int row_chunks = (int)(row_bytes / 16);
    const unsigned grid = (unsigned)((rows_cap + 3) / 4);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(tr_gather_rows_kernel, dim3(grid), dim3(256), 0, s, static_cast<const u32x4*>(X), row_chunks,
                       T, row_tok, offsets_r, E, rows_cap, static_cast<u32x4*>(Xp));
    return hipGetLastError();
}

}  // namespace moe
