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
constexpr int kBins = 256;  // radix digit of 8 bits
// Lanes count into kSub copies of the histogram (lane % kSub), each padded by
// one word so that the copies of a bin sit in different banks: normal logits
// put nearly every key's top byte into a few bins, and lanes adding to one
// LDS word serialise.
constexpr int kSub = 16, kSubLd = kBins + 1, kHistWords = kSub * kSubLd;
constexpr int kSelBatch = 16;  // tokens a thread loads at once (kept for every pass when T <= 16384)

// Flags and keys of tokens [b0, b0 + kSelBatch) that lie below t_hi; flag 0xFF
// (neither routed nor not routed) past t_hi.  All loads are issued together.
MOE_DEV void sel_load(const uint8_t* __restrict__ mem, const uint32_t* __restrict__ key, int b0, int t_hi,
                      uint8_t (&mm)[kSelBatch], uint32_t (&kk)[kSelBatch]) {
#pragma unroll
    for (int j = 0; j < kSelBatch; ++j) {
        const int t = b0 + j;
        const bool v = t < t_hi;
        mm[j] = v ? mem[t] : (uint8_t)0xFF;
        kk[j] = v ? key[t] : 0u;
    }
}

// Exclusive prefix sum of a 64-bit value over the workgroup in thread order;
// *total gets the workgroup's sum.  Every thread must call it.
MOE_DEV long long block_excl_scan_ll(long long v, long long* s_ll, long long* total) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    long long x = v;
#pragma unroll
    for (int s = 1; s < kWave; s <<= 1) {
        const long long y = __shfl_up(x, s, kWave);
        if (lane >= s) x += y;
    }
    if (lane == kWave - 1) s_ll[wave] = x;
    __syncthreads();
    // lanes 0..15 hold the wave totals; sum those before this wave, and all
    const long long wt = lane < kSelWaves ? s_ll[lane] : 0;
    long long before = lane < wave ? wt : 0, tot = wt;
#pragma unroll
    for (int s = 1; s < kSelWaves; s <<= 1) {
        before += __shfl_xor(before, s, kWave);
        tot += __shfl_xor(tot, s, kWave);
    }
    before = __shfl(before, 0, kWave);
    tot = __shfl(tot, 0, kWave);
    __syncthreads();
    *total = tot;
    return before + x - v;
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

// LDS staging of an expert's keys and flags when T <= 16384 (one batch per
// thread): global memory is read and written in token order across threads
// (coalesced), and each thread reads its own run of tokens from LDS.  One pad
// word (keys) or 4 pad bytes (flags) after every 16 tokens spread a thread's
// run over distinct banks.
constexpr int kSelStageT = kSelThreads * kSelBatch;
constexpr int kStageKeyWords = kSelStageT + kSelStageT / 16;
constexpr int kStageMemBytes = kSelStageT + kSelStageT / 4;
constexpr size_t kSelLds = (size_t)kStageKeyWords * 4 + kStageMemBytes;
MOE_DEV int skw(int t) { return t + (t >> 4); }
MOE_DEV int skb(int t) { return t + ((t >> 4) << 2); }

// One workgroup per expert e.  counts[] is the histogram of topk_idx (as
// moe_route writes it); rows of e are [o, o + r) with o the sum of the targets
// of the experts before e.  Writes counts_r[e], offsets_r[e] (and offsets_r[E]
// from the last expert), row_tok[o .. o+r) and slotT[e*T + t] for every t.
// Nothing is written past rows_cap rows, whatever counts holds.
// Thread i owns the contiguous tokens [i*c, (i+1)*c), c = ceil(T / 1024), so
// thread order is token order and one scan over threads ranks the kept tokens.
__global__ __launch_bounds__(kSelThreads) void tr_select_kernel(
    const uint32_t* __restrict__ keyT, const uint8_t* __restrict__ memT, int T, int E, int M, int cap_tiles,
    const int32_t* __restrict__ counts, int32_t* __restrict__ counts_r, int32_t* __restrict__ offsets_r,
    int32_t* __restrict__ row_tok, long long rows_cap, int32_t* __restrict__ slotT) {
    extern __shared__ __attribute__((aligned(16))) char sel_stage[];  // kSelLds bytes when T <= kSelStageT
    __shared__ int s_hist[2][kHistWords];
    __shared__ int s_scan[kBins];
    __shared__ long long s_ll[kSelWaves];
    __shared__ int s_digit, s_above, s_total;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int e = blockIdx.x;
    const uint32_t* key = keyT + (size_t)e * T;
    const uint8_t* mem = memT + (size_t)e * T;
    int32_t* srow = slotT + (size_t)e * T;
    const int c = (T + kSelThreads - 1) / kSelThreads;
    const int t_lo = min(tid * c, T), t_hi = min(t_lo + c, T);
    // Each thread's tokens, loaded once when they fit one batch (c is uniform),
    // through LDS: coalesced global loads, then each thread's run.
    const bool cached = c <= kSelBatch;
    uint32_t* s_key = reinterpret_cast<uint32_t*>(sel_stage);
    uint8_t* s_mem = reinterpret_cast<uint8_t*>(sel_stage + (size_t)kStageKeyWords * 4);
    uint8_t mm[kSelBatch];
    uint32_t kk[kSelBatch];
    if (cached) {
#pragma unroll
        for (int j = 0; j < kSelBatch; ++j) {
            const int q = j * kSelThreads + tid;
            const bool v = q < T;
            kk[j] = v ? key[q] : 0u;
            mm[j] = v ? mem[q] : (uint8_t)0xFF;
        }
#pragma unroll
        for (int j = 0; j < kSelBatch; ++j) {
            const int q = j * kSelThreads + tid;
            if (q < T) {
                s_key[skw(q)] = kk[j];
                s_mem[skb(q)] = mm[j];
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kSelBatch; ++j) {
            const int t = t_lo + j;
            const bool v = t < t_hi;
            kk[j] = v ? s_key[skw(t)] : 0u;
            mm[j] = v ? s_mem[skb(t)] : (uint8_t)0xFF;
        }
    }

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
        for (int q = tid; q < kHistWords; q += kSelThreads) s_hist[0][q] = 0;
        __syncthreads();
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            int* hist = s_hist[pass & 1];
            int* my_hist = hist + (lane & (kSub - 1)) * kSubLd;
            for (int q = tid; q < kHistWords; q += kSelThreads) s_hist[(pass + 1) & 1][q] = 0;  // next pass
            for (int b0 = t_lo; b0 < t_hi; b0 += kSelBatch) {
                if (!cached) sel_load(mem, key, b0, t_hi, mm, kk);
#pragma unroll
                for (int j = 0; j < kSelBatch; ++j)
                    if (mm[j] == want && (kk[j] & hmask) == prefix)
                        atomicAdd(&my_hist[(kk[j] >> shift) & (kBins - 1)], 1);
            }
            __syncthreads();
            // above(b) = candidates in bins above b: an inclusive scan from the
            // top bin down, 64 bins per wave, then the totals of the waves before.
            int v = 0;
            if (tid < kBins) {
#pragma unroll
                for (int u = 0; u < kSub; ++u) v += hist[u * kSubLd + kBins - 1 - tid];
                int x = v;
#pragma unroll
                for (int s = 1; s < kWave; s <<= 1) {
                    const int y = __shfl_up(x, s, kWave);
                    if (lane >= s) x += y;
                }
                s_scan[tid] = x;
            }
            __syncthreads();
            if (tid < kBins) {
                int incl = s_scan[tid];
                for (int w = 0; w < wave; ++w) incl += s_scan[w * kWave + kWave - 1];
                const int above = incl - v;
                if (above < need && need <= incl) {
                    s_digit = kBins - 1 - tid;
                    s_above = above;
                }
                if (tid == kBins - 1) s_total = incl;
            }
            __syncthreads();
            if (pass == 0 && s_total <= need) {
                take_all = true;
                break;
            }
            prefix |= (uint32_t)s_digit << shift;
            hmask |= 0xFFu << shift;
            need -= s_above;
        }
        tau = prefix;
    }

    // Kept tokens in ascending order.  Per thread: ties with tau (taken in
    // token order while fewer than `need` came before) and the other kept
    // tokens; one scan of both counts gives each thread its first tie rank and
    // its first row.
    int n_tie = 0, n_sel = 0;
    for (int b0 = t_lo; b0 < t_hi; b0 += kSelBatch) {
        if (!cached) sel_load(mem, key, b0, t_hi, mm, kk);
#pragma unroll
        for (int j = 0; j < kSelBatch; ++j) {
            const bool cand = m > 0 && mm[j] == want;
            const bool always = !down && mm[j] == 1;
            if (cand && !take_all) {
                n_tie += kk[j] == tau;
                n_sel += kk[j] > tau;
            } else {
                n_sel += always || cand;
            }
        }
    }
    long long tot2;
    const long long base2 = block_excl_scan_ll(((long long)n_tie << 32) | (long long)n_sel, s_ll, &tot2);
    int tie_rank = (int)(base2 >> 32);
    int pos = (int)(base2 & 0xFFFFFFFFll) + min(tie_rank, need);
    for (int b0 = t_lo; b0 < t_hi; b0 += kSelBatch) {
        if (!cached) sel_load(mem, key, b0, t_hi, mm, kk);
#pragma unroll
        for (int j = 0; j < kSelBatch; ++j) {
            const int t = b0 + j;
            if (t >= t_hi) break;
            const bool cand = m > 0 && mm[j] == want;
            const bool always = !down && mm[j] == 1;
            bool sel;
            if (cand && !take_all) {
                const bool tie = kk[j] == tau;
                sel = kk[j] > tau || (tie && tie_rank < need);
                tie_rank += tie;
            } else {
                sel = always || cand;
            }
            int32_t row = -1;
            if (sel) {
                if (room && pos < r) {
                    row = (int32_t)(o + pos);
                    row_tok[row] = t;
                }
                ++pos;
            }
            if (cached) s_key[skw(t)] = (uint32_t)row;  // every read of s_key was before the scan's barriers
            else srow[t] = row;
        }
    }
    if (cached) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kSelBatch; ++j) {
            const int q = j * kSelThreads + tid;
            if (q < T) srow[q] = (int32_t)s_key[skw(q)];
        }
    }
}

constexpr int kSlotTokens = 32;                 // tokens per workgroup of tr_slots_kernel
constexpr int kSlotPerWave = kSlotTokens / 4;   // tokens per wave
constexpr int kSlotMaxE = 256;                  // experts per token held in registers (4 per lane)

// slot_row[t,e] from slotT[e,t] (through LDS), and slot_w[t,e] = softmax of
// logits[t,:] over the kept experts: exp(l - m) / sum, m the largest kept
// logit, fp32; 0 where not kept.  One wave per token, 8 tokens per wave; the
// logits of all 8 are loaded before the first is reduced.  E <= 256.
__global__ __launch_bounds__(256) void tr_slots_kernel(const float* __restrict__ logits,
                                                       const int32_t* __restrict__ slotT, int T, int E,
                                                       int32_t* __restrict__ slot_row, float* __restrict__ slot_w) {
    constexpr int NE = kSlotMaxE / kWave;
    extern __shared__ int32_t s_rows[];  // [kSlotTokens][E + 1]
    const int t0 = blockIdx.x * kSlotTokens;
    const int ld = E + 1;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    float lv[kSlotPerWave][NE];
#pragma unroll
    for (int j = 0; j < kSlotPerWave; ++j) {
        const int t = t0 + wave * kSlotPerWave + j;
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            const int e = lane + i * kWave;
            lv[j][i] = (t < T && e < E) ? logits[(size_t)t * E + e] : 0.0f;
        }
    }
    // slotT entries of the 32 tokens (at most 32 per thread), all loads issued together
    constexpr int NQ = kSlotTokens * kSlotMaxE / 256;
    int32_t rv[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const int q = threadIdx.x + 256 * i;
        const int e = q / kSlotTokens, t = t0 + q % kSlotTokens;
        rv[i] = (e < E && t < T) ? slotT[(size_t)e * T + t] : -1;
    }
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const int q = threadIdx.x + 256 * i;
        const int e = q / kSlotTokens, tt = q % kSlotTokens;
        if (e < E) s_rows[tt * ld + e] = rv[i];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSlotPerWave; ++j) {
        const int tt = wave * kSlotPerWave + j;
        const int t = t0 + tt;
        if (t >= T) break;
        int32_t row[NE];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            const int e = lane + i * kWave;
            row[i] = e < E ? s_rows[tt * ld + e] : -1;
            if (row[i] >= 0) mx = fmaxf(mx, lv[j][i]);
        }
        mx = group_max<kWave>(mx);
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < NE; ++i)
            if (row[i] >= 0) sum += expf(lv[j][i] - mx);
        sum = group_sum<kWave>(sum);
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            const int e = lane + i * kWave;
            if (e < E) {
                slot_row[(size_t)t * E + e] = row[i];
                slot_w[(size_t)t * E + e] = row[i] >= 0 ? expf(lv[j][i] - mx) / sum : 0.0f;
            }
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
    const size_t sel_lds = T <= kSelStageT ? kSelLds : 0;
    if (sel_lds != 0) {
        const hipError_t aerr =
            hipFuncSetAttribute((const void*)tr_select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSelLds);
        if (aerr != hipSuccess) return aerr;
    }
    hipLaunchKernelGGL(tr_select_kernel, dim3((unsigned)E), dim3(kSelThreads), sel_lds, s, keyT, memT, T, E, M,
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
