// C ABI of libmoe: argument validation, workspace carving and kernel
// orchestration for the MoE layer forward and its data-gradient backward.  The entry points are declared
// (with their semantics and the passages they follow) in include/moe.h.
#include "../../include/moe.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "launch.h"

namespace moe {

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMaxE = 256;
constexpr int kMaxK = 8;

// Shared checks of (T, E, K).  Returns MOE_OK or an error status.
int check_tek(int T, int E, int K) {
    if (T < 1) return fail(MOE_ERR_INVALID_ARG, "T must be >= 1 (got %d)", T);
    if (E < 1) return fail(MOE_ERR_INVALID_ARG, "E must be >= 1 (got %d)", E);
    if (K < 1 || K > E) return fail(MOE_ERR_INVALID_ARG, "K must be in [1, E] (got K=%d, E=%d)", K, E);
    if (E > kMaxE) return fail(MOE_ERR_UNSUPPORTED, "E=%d exceeds the supported maximum %d", E, kMaxE);
    if (K > kMaxK) return fail(MOE_ERR_UNSUPPORTED, "K=%d exceeds the supported maximum %d", K, kMaxK);
    if ((long long)T * K >= (1LL << 31)) return fail(MOE_ERR_UNSUPPORTED, "T*K must be < 2^31");
    return MOE_OK;
}

int check_dtype(int dtype) {
    if (dtype != MOE_F32 && dtype != MOE_BF16)
        return fail(MOE_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
    return MOE_OK;
}

size_t elem_bytes(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

// Feature dimensions handled by the tile kernels: multiples of the tile edge.
int check_dim(const char* name, int v, int dtype) {
    const int q = dtype == MOE_BF16 ? 128 : 64;
    if (v < 1) return fail(MOE_ERR_INVALID_ARG, "%s must be >= 1 (got %d)", name, v);
    if (v % q != 0)
        return fail(MOE_ERR_UNSUPPORTED, "%s=%d must be a multiple of %d for this dtype", name, v, q);
    return MOE_OK;
}

// Row-copy dims: 16-byte rows suffice.
int check_row(int d, int dtype) {
    if (d < 1) return fail(MOE_ERR_INVALID_ARG, "d must be >= 1 (got %d)", d);
    if (((size_t)d * elem_bytes(dtype)) % 16 != 0)
        return fail(MOE_ERR_UNSUPPORTED, "rows of d=%d elements must be a multiple of 16 bytes", d);
    return MOE_OK;
}

#define CHECK(expr)                     \
    do {                                \
        const int _s = (expr);          \
        if (_s != MOE_OK) return _s;    \
    } while (0)

#define NONNULL(p)                                                                          \
    do {                                                                                    \
        if ((p) == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s must not be NULL", #p);     \
        if (!aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "%s must be 16-byte aligned", #p); \
    } while (0)

#define HIPCHECK(expr)                                                                       \
    do {                                                                                     \
        const hipError_t _e = (expr);                                                        \
        if (_e != hipSuccess)                                                                \
            return fail(MOE_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(_e));         \
    } while (0)

// Workspace carving: a bump allocator over the caller's buffer.
struct Carver {
    char* base;
    size_t used = 0;
    explicit Carver(void* b) : base(static_cast<char*>(b)) {}
    template <typename T>
    T* take(size_t count) {
        T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
        used += align_up(count * sizeof(T));
        return p;
    }
};

size_t route_ws(int T, int E) { return align_up((size_t)num_chunks(T) * E * sizeof(int32_t)); }

size_t permute_ws(int T, int E) {
    return 2 * align_up((size_t)num_chunks(T) * E * sizeof(int32_t)) + align_up(E * sizeof(int32_t)) +
           align_up((E + 1) * sizeof(int32_t));
}

// sub_tokens: tokens per row of the expert histogram (0: chunk_tokens(T)).
size_t forward_ws(int T, int d, int E, int K, int n, int dtype, int sub_tokens = 0) {
    const size_t A = (size_t)T * K;
    const size_t s = elem_bytes(dtype);
    size_t b = 0;
    b += 2 * align_up((size_t)count_rows(T, sub_tokens) * E * 4);  // blk, blkbase
    b += align_up(A * 4) * 2;                          // topk_idx, topk_w
    b += align_up(E * 4) + align_up((E + 1) * 4);      // counts, offsets
    b += align_up(A * 4) * 2;                          // sorted_pair, inv
    // Xp only where the SwiGLU GEMM cannot gather the X rows itself
    b += (ffn_gather_ok(dtype, T, d, n) ? 0 : align_up(A * d * s)) + align_up(A * d * s) + align_up(A * n * s);  // Xp, Y, Act
    b += align_up(ffn_split_bytes(dtype, d, n));        // split tail of the grouped GEMMs
    return b;
}

// The router front end of the calls that start from X (moe_route_x,
// moe_forward_x): the bf16 split of Wr, then room for the logits where the
// projection is not fused with the gate.  Tokens per histogram row after it.
bool route_x_fused(int dtype, int d, int E) { return router_gate_ok(dtype, d, E); }
int route_x_rows_tokens(int dtype, int d, int E) { return route_x_fused(dtype, d, E) ? kRouterGateTokens : 0; }
size_t route_x_front_ws(int T, int d, int E, int dtype) {
    size_t b = align_up(router_split_bytes(dtype, d, E));
    if (!route_x_fused(dtype, d, E)) b += align_up((size_t)T * E * 4);
    return b;
}

// Checks of the router arguments shared by moe_router and the calls from X.
int check_router(int T, int d, int E) {
    if (T < 1) return fail(MOE_ERR_INVALID_ARG, "T must be >= 1 (got %d)", T);
    if (d < 1) return fail(MOE_ERR_INVALID_ARG, "d must be >= 1 (got %d)", d);
    if (E < 1) return fail(MOE_ERR_INVALID_ARG, "E must be >= 1 (got %d)", E);
    if (E > kMaxE) return fail(MOE_ERR_UNSUPPORTED, "E=%d exceeds the supported maximum %d", E, kMaxE);
    if ((long long)T * E >= (1LL << 31)) return fail(MOE_ERR_UNSUPPORTED, "T*E must be < 2^31");
    return MOE_OK;
}

// Workspace of moe_backward_data, in carving order.
size_t backward_ws(int T, int d, int E, int K, int n, int dtype, bool weights) {
    const size_t A = (size_t)T * K;
    const size_t s = elem_bytes(dtype);
    size_t b = 0;
    b += 2 * align_up((size_t)num_chunks(T) * E * 4);       // blk, blkbase
    b += align_up(A * 4) * 2;                               // topk_idx, topk_w
    b += align_up(E * 4) + align_up((E + 1) * 4);           // counts, offsets
    b += align_up(A * 4) * 2;                               // sorted_pair, inv
    b += align_up(A * 4) * 2;                               // dS, unit weights
    b += align_up(A * d * s) * 2;                           // Xp (then dXp), dout rows
    b += align_up(2 * A * n * s) + align_up(A * n * s) + align_up(A * 2 * n * s);  // H1|H3, dA, dH
    if (!ffn_bt_ok(dtype, n, d, d)) b += align_up((size_t)E * d * n * s);          // W2^T
    if (!ffn_bt_ok(dtype, d, 2 * n, n)) b += align_up((size_t)E * 2 * d * n * s);  // [W1^T ; W3^T]
    b += align_up(ffn_split_bytes(dtype, 256, 128));        // split tail of the grouped GEMMs
    if (weights) b += align_up(A * n * s);                  // w * act, for dW2
    return b;
}

// Optional split workspace of the grouped GEMMs: NULL disables the split.
int ffn_split_arg(void* ws, size_t ws_bytes, int dtype, int d, int n, float** part) {
    *part = nullptr;
    if (ws == nullptr) return MOE_OK;
    const size_t need = ffn_split_bytes(dtype, d, n);
    if (need == 0) return MOE_OK;
    if (ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "the grouped GEMM workspace needs %zu bytes (got %zu)", need, ws_bytes);
    if (!aligned16(ws)) return fail(MOE_ERR_INVALID_ARG, "ws must be 16-byte aligned");
    *part = static_cast<float*>(ws);
    return MOE_OK;
}

// Token Rounding arguments: (T, E, K) as for routing, tile rows M, limit in tiles.
int check_tr(int T, int E, int K, int M, int cap_tiles) {
    CHECK(check_tek(T, E, K));
    if (M < 1) return fail(MOE_ERR_INVALID_ARG, "M must be >= 1 (got %d)", M);
    if (M > 65536) return fail(MOE_ERR_UNSUPPORTED, "M=%d exceeds the supported maximum 65536", M);
    if (cap_tiles < 0) return fail(MOE_ERR_INVALID_ARG, "cap_tiles must be >= 0 (got %d)", cap_tiles);
    if ((long long)T * E >= (1LL << 31)) return fail(MOE_ERR_UNSUPPORTED, "T*E must be < 2^31");
    return MOE_OK;
}

// Most rows a Token Rounding plan can have: an expert rounds up by at most
// floor(M/2) rows and never holds a token twice.
long long tr_max_rows(int T, int E, int K, int M) {
    const long long a = (long long)T * K + (long long)E * (M / 2);
    const long long b = (long long)T * E;
    return a < b ? a : b;
}

size_t forward_tr_ws(int T, int d, int E, int K, int n, int M, int dtype) {
    const size_t A = (size_t)T * K;
    const size_t R = (size_t)tr_max_rows(T, E, K, M);
    const size_t s = elem_bytes(dtype);
    size_t b = 0;
    b += 2 * align_up((size_t)num_chunks(T) * E * 4);  // blk, blkbase
    b += align_up(A * 4) * 2;                          // topk_idx, topk_w
    b += align_up(E * 4) + align_up((E + 1) * 4);      // counts, offsets
    b += align_up(tr_keys_bytes(T, E));                // keys, flags and rows by expert
    b += align_up(E * 4) + align_up((E + 1) * 4);      // counts_r, offsets_r
    b += align_up(R * 4);                              // row_tok
    b += align_up((size_t)T * E * 4) * 2;              // slot_row, slot_w
    b += (ffn_gather_ok(dtype, T, d, n) ? 0 : align_up(R * d * s)) + align_up(R * d * s) + align_up(R * n * s);
    b += align_up(ffn_split_bytes(dtype, d, n));
    return b;
}

std::atomic<int> g_cu_count[64];

// Scratch of moe_route_noalloc: the gate's per-chunk expert counts, in a
// file-scope device array that every GPU the library runs on holds until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it only names a stand-in, not device memory): the array's address on
// each device is looked up once, with that device current, and kept here.
constexpr size_t kNoAllocScratchInts = MOE_ROUTE_NOALLOC_SCRATCH_BYTES / sizeof(int32_t);
__device__ __align__(256) int32_t scratch[kNoAllocScratchInts];

constexpr int kMaxDevices = 64;
std::atomic<int32_t*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// This device's address of `scratch`, looked up on the first call on the
// device; MOE_OK or an error status.
int noalloc_scratch(int32_t** out) {
    int dev = -1;
    const hipError_t derr = hipGetDevice(&dev);
    if (derr != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(derr));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MOE_ERR_UNSUPPORTED, "device %d is beyond the %d devices the scratch table covers", dev,
                    kMaxDevices);
    int32_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            void* addr = nullptr;
            const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
            if (e != hipSuccess || addr == nullptr)
                return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                            hipGetErrorString(e));
            p = static_cast<int32_t*>(addr);
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MOE_OK;
}

}  // namespace

int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int c = g_cu_count[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
        cu = 256;
    if (dev < 64) g_cu_count[dev].store(cu, std::memory_order_relaxed);
    return cu;
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported size or dtype";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* moe_last_error(void) { return g_last_error; }

size_t moe_workspace_bytes(int T, int d, int E, int K, int n, int dtype) {
    if (check_tek(T, E, K) != MOE_OK || check_dtype(dtype) != MOE_OK || check_dim("d", d, dtype) != MOE_OK ||
        check_dim("n", n, dtype) != MOE_OK)
        return 0;
    size_t b = forward_ws(T, d, E, K, n, dtype);
    for (const size_t x : {route_ws(T, E), permute_ws(T, E), ffn_split_bytes(dtype, d, n)}) b = x > b ? x : b;
    return b;
}

size_t moe_route_workspace_bytes(int T, int E, int K) {
    if (check_tek(T, E, K) != MOE_OK) return 0;
    return route_ws(T, E);
}

size_t moe_permute_workspace_bytes(int T, int E, int K) {
    if (check_tek(T, E, K) != MOE_OK) return 0;
    return permute_ws(T, E);
}

size_t moe_ffn_workspace_bytes(int d, int n, int dtype) {
    if (check_dtype(dtype) != MOE_OK || check_dim("d", d, dtype) != MOE_OK || check_dim("n", n, dtype) != MOE_OK)
        return 0;
    return ffn_split_bytes(dtype, d, n);
}

size_t moe_router_workspace_bytes(int d, int E, int dtype) {
    if (check_dtype(dtype) != MOE_OK || d < 1 || E < 1 || E > kMaxE) return 0;
    return router_split_bytes(dtype, d, E);
}

size_t moe_forward_workspace_bytes(int T, int d, int E, int K, int n, int dtype) {
    if (check_tek(T, E, K) != MOE_OK || check_dtype(dtype) != MOE_OK || check_dim("d", d, dtype) != MOE_OK ||
        check_dim("n", n, dtype) != MOE_OK)
        return 0;
    return forward_ws(T, d, E, K, n, dtype);
}

int moe_route(const float* logits, int T, int E, int K, int32_t* topk_idx, float* topk_w,
              int32_t* counts, int32_t* offsets, void* ws, size_t ws_bytes, void* stream) {
    CHECK(check_tek(T, E, K));
    NONNULL(logits);
    NONNULL(topk_idx);
    NONNULL(topk_w);
    NONNULL(counts);
    NONNULL(offsets);
    const size_t need = route_ws(T, E);
    if (ws == nullptr || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "moe_route needs %zu workspace bytes (got %zu)", need, ws_bytes);
    if (!aligned16(ws)) return fail(MOE_ERR_INVALID_ARG, "ws must be 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    Carver c(ws);
    int32_t* blk = c.take<int32_t>((size_t)num_chunks(T) * E);
    HIPCHECK(launch_gate(logits, T, E, K, topk_idx, topk_w, blk, s));
    HIPCHECK(launch_scan(blk, num_chunks(T), E, counts, offsets, nullptr, s));
    return MOE_OK;
}

int moe_route_noalloc(const float* logits, int T, int E, int K, int32_t* topk_idx, float* topk_w, int32_t* counts,
                      int32_t* offsets, void* stream) {
    CHECK(check_tek(T, E, K));
    NONNULL(logits);
    NONNULL(topk_idx);
    NONNULL(topk_w);
    NONNULL(counts);
    NONNULL(offsets);
    const size_t need = (size_t)num_chunks(T) * E;
    if (need > kNoAllocScratchInts)
        return fail(MOE_ERR_UNSUPPORTED,
                    "moe_route_noalloc: %d chunks of %d tokens x E=%d need %zu bytes of scratch, above its %zu",
                    num_chunks(T), chunk_tokens(T), E, need * sizeof(int32_t), (size_t)MOE_ROUTE_NOALLOC_SCRATCH_BYTES);
    int32_t* blk = nullptr;
    CHECK(noalloc_scratch(&blk));
    hipStream_t s = static_cast<hipStream_t>(stream);
    // The gate writes every chunk's E counts before the scan reads them, so
    // what an earlier call left in the scratch is never read.
    HIPCHECK(launch_gate(logits, T, E, K, topk_idx, topk_w, blk, s));
    HIPCHECK(launch_scan(blk, num_chunks(T), E, counts, offsets, nullptr, s));
    return MOE_OK;
}

int moe_permute(const void* X, int dtype, int T, int d, int E, int K, const int32_t* topk_idx,
                int32_t* sorted_pair, int32_t* inv, void* Xp, void* ws, size_t ws_bytes, void* stream) {
    CHECK(check_tek(T, E, K));
    CHECK(check_dtype(dtype));
    CHECK(check_row(d, dtype));
    NONNULL(X);
    NONNULL(topk_idx);
    NONNULL(sorted_pair);
    NONNULL(inv);
    NONNULL(Xp);
    const size_t need = permute_ws(T, E);
    if (ws == nullptr || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "moe_permute needs %zu workspace bytes (got %zu)", need, ws_bytes);
    if (!aligned16(ws)) return fail(MOE_ERR_INVALID_ARG, "ws must be 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int B = num_chunks(T);
    Carver c(ws);
    int32_t* blk = c.take<int32_t>((size_t)B * E);
    int32_t* blkbase = c.take<int32_t>((size_t)B * E);
    int32_t* cnt = c.take<int32_t>(E);
    int32_t* off = c.take<int32_t>(E + 1);
    HIPCHECK(launch_chunk_hist(topk_idx, T, E, K, blk, s));
    if (scan_rank_fused(T, E)) {
        HIPCHECK(launch_scan_rank(topk_idx, T, E, K, blk, nullptr, nullptr, sorted_pair, inv, nullptr, 0, s));
    } else {
        HIPCHECK(launch_scan(blk, B, E, cnt, off, blkbase, s));
        HIPCHECK(launch_rank(topk_idx, T, E, K, blkbase, sorted_pair, inv, s));
    }
    HIPCHECK(launch_copy_rows(X, (size_t)d * elem_bytes(dtype), T, K, inv, Xp, s));
    return MOE_OK;
}

int moe_grouped_ffn(const void* Xp, const void* W1, const void* W3, const void* W2, int dtype, int T,
                    int d, int E, int K, int n, const int32_t* counts, const int32_t* offsets, void* Act,
                    void* Y, void* ws, size_t ws_bytes, void* stream) {
    CHECK(check_tek(T, E, K));
    CHECK(check_dtype(dtype));
    CHECK(check_dim("d", d, dtype));
    CHECK(check_dim("n", n, dtype));
    NONNULL(Xp);
    NONNULL(W1);
    NONNULL(W3);
    NONNULL(W2);
    NONNULL(counts);
    NONNULL(offsets);
    NONNULL(Act);
    NONNULL(Y);
    if ((long long)T * K * (long long)(d > n ? d : n) >= (1LL << 40))
        return fail(MOE_ERR_UNSUPPORTED, "T*K*max(d,n) must be < 2^40");
    float* part = nullptr;
    CHECK(ffn_split_arg(ws, ws_bytes, dtype, d, n, &part));
    HIPCHECK(launch_ffn(Xp, W1, W3, W2, dtype, T * K, d, E, n, counts, offsets, Act, Y, part, false,
                        static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

int moe_ffn_up(const void* Xp, const void* W1, const void* W3, int dtype, int T, int d, int E, int K, int n,
               const int32_t* counts, const int32_t* offsets, void* Act, void* ws, size_t ws_bytes,
               void* stream) {
    CHECK(check_tek(T, E, K));
    CHECK(check_dtype(dtype));
    CHECK(check_dim("d", d, dtype));
    CHECK(check_dim("n", n, dtype));
    NONNULL(Xp);
    NONNULL(W1);
    NONNULL(W3);
    NONNULL(counts);
    NONNULL(offsets);
    NONNULL(Act);
    if ((long long)T * K * (long long)(d > n ? d : n) >= (1LL << 40))
        return fail(MOE_ERR_UNSUPPORTED, "T*K*max(d,n) must be < 2^40");
    float* part = nullptr;
    CHECK(ffn_split_arg(ws, ws_bytes, dtype, d, n, &part));
    HIPCHECK(launch_ffn_up(Xp, W1, W3, dtype, T * K, d, E, n, counts, offsets, Act, part, false,
                           static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

int moe_ffn_down(const void* Act, const void* W2, int dtype, int T, int d, int E, int K, int n,
                 const int32_t* counts, const int32_t* offsets, void* Y, void* ws, size_t ws_bytes,
                 void* stream) {
    CHECK(check_tek(T, E, K));
    CHECK(check_dtype(dtype));
    CHECK(check_dim("d", d, dtype));
    CHECK(check_dim("n", n, dtype));
    NONNULL(Act);
    NONNULL(W2);
    NONNULL(counts);
    NONNULL(offsets);
    NONNULL(Y);
    if ((long long)T * K * (long long)(d > n ? d : n) >= (1LL << 40))
        return fail(MOE_ERR_UNSUPPORTED, "T*K*max(d,n) must be < 2^40");
    float* part = nullptr;
    CHECK(ffn_split_arg(ws, ws_bytes, dtype, d, n, &part));
    HIPCHECK(launch_ffn_down(Act, W2, dtype, T * K, d, E, n, counts, offsets, Y, part, false,
                             static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

int moe_router(const void* X, int dtype, int T, int d, int E, const float* Wr, const float* bias,
               float* logits, void* ws, size_t ws_bytes, void* stream) {
    CHECK(check_router(T, d, E));
    CHECK(check_dtype(dtype));
    NONNULL(X);
    NONNULL(Wr);
    NONNULL(logits);
    const size_t need = router_split_bytes(dtype, d, E);
    if (need > 0) {
        if (ws == nullptr || ws_bytes < need)
            return fail(MOE_ERR_WORKSPACE, "moe_router needs %zu workspace bytes (got %zu)", need, ws_bytes);
        if (!aligned16(ws) || !aligned16(X)) return fail(MOE_ERR_INVALID_ARG, "X and ws must be 16-byte aligned");
    }
    HIPCHECK(launch_router(X, dtype, T, d, E, Wr, bias, logits, need > 0 ? ws : nullptr,
                           static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

int moe_combine(const void* Y, const float* topk_w, const int32_t* inv, int dtype, int T, int d, int K,
                void* out, void* stream) {
    if (T < 1) return fail(MOE_ERR_INVALID_ARG, "T must be >= 1 (got %d)", T);
    if (K < 1) return fail(MOE_ERR_INVALID_ARG, "K must be >= 1 (got %d)", K);
    if (K > kMaxK) return fail(MOE_ERR_UNSUPPORTED, "K=%d exceeds the supported maximum %d", K, kMaxK);
    if ((long long)T * K >= (1LL << 31)) return fail(MOE_ERR_UNSUPPORTED, "T*K must be < 2^31");
    CHECK(check_dtype(dtype));
    CHECK(check_row(d, dtype));
    NONNULL(Y);
    NONNULL(topk_w);
    NONNULL(inv);
    NONNULL(out);
    HIPCHECK(launch_combine(Y, topk_w, inv, dtype, T, d, K, out, static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

size_t moe_route_x_workspace_bytes(int T, int d, int E, int K, int dtype) {
    if (check_tek(T, E, K) != MOE_OK || check_router(T, d, E) != MOE_OK || check_dtype(dtype) != MOE_OK) return 0;
    return route_x_front_ws(T, d, E, dtype) +
           align_up((size_t)count_rows(T, route_x_rows_tokens(dtype, d, E)) * E * sizeof(int32_t));
}

size_t moe_forward_x_workspace_bytes(int T, int d, int E, int K, int n, int dtype) {
    if (check_tek(T, E, K) != MOE_OK || check_router(T, d, E) != MOE_OK || check_dtype(dtype) != MOE_OK ||
        check_dim("d", d, dtype) != MOE_OK || check_dim("n", n, dtype) != MOE_OK)
        return 0;
    return route_x_front_ws(T, d, E, dtype) + forward_ws(T, d, E, K, n, dtype, route_x_rows_tokens(dtype, d, E));
}

}  // extern "C"

namespace {

// Steps 0-1 of the calls from X into topk_idx / topk_w and the expert counts
// blk (rows of route_x_rows_tokens() tokens): fused where route_x_fused(),
// else moe_router's kernels into `lg` (the caller's logits or workspace room)
// and the gate.  `front` is the workspace part route_x_front_ws() sizes.
int route_x_front(const void* X, int dtype, int T, int d, int E, int K, const float* Wr, const float* bias,
                  float* logits, int32_t* topk_idx, float* topk_w, int32_t* blk, void* front, hipStream_t s) {
    Carver c(front);
    void* split = c.take<char>(router_split_bytes(dtype, d, E));
    if (route_x_fused(dtype, d, E)) {
        HIPCHECK(launch_router_gate(X, T, d, E, K, Wr, bias, logits, topk_idx, topk_w, blk, split, s));
    } else {
        float* room = c.take<float>((size_t)T * E);
        float* lg = logits != nullptr ? logits : room;
        HIPCHECK(launch_router(X, dtype, T, d, E, Wr, bias, lg, router_split_bytes(dtype, d, E) ? split : nullptr, s));
        HIPCHECK(launch_gate(lg, T, E, K, topk_idx, topk_w, blk, s));
    }
    return MOE_OK;
}

// moe_forward (logits given) and moe_forward_x (Wr given: the router runs
// first, fused with the gate where it can be).
int forward_impl(const char* name, const void* X, const float* logits_in, const float* Wr, const float* bias,
                 float* logits_out, const void* W1, const void* W3, const void* W2, int dtype, int T, int d, int E,
                 int K, int n, void* out, int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                 int32_t* sorted_pair, int32_t* inv, void* ws, size_t ws_bytes, void* stream) {
    const bool from_x = Wr != nullptr;
    CHECK(check_tek(T, E, K));
    CHECK(check_dtype(dtype));
    CHECK(check_dim("d", d, dtype));
    CHECK(check_dim("n", n, dtype));
    NONNULL(X);
    if (!from_x) NONNULL(logits_in);
    if (from_x) CHECK(check_router(T, d, E));
    NONNULL(W1);
    NONNULL(W3);
    NONNULL(W2);
    NONNULL(out);
    for (const void* p : {(const void*)topk_idx, (const void*)topk_w, (const void*)counts, (const void*)offsets,
                          (const void*)sorted_pair, (const void*)inv, (const void*)logits_out, (const void*)bias})
        if (p != nullptr && !aligned16(p))
            return fail(MOE_ERR_INVALID_ARG, "optional arguments must be 16-byte aligned");
    if ((long long)T * K * (long long)(d > n ? d : n) >= (1LL << 40))
        return fail(MOE_ERR_UNSUPPORTED, "T*K*max(d,n) must be < 2^40");
    const int st = from_x ? route_x_rows_tokens(dtype, d, E) : 0;  // tokens per histogram row
    const size_t front = from_x ? route_x_front_ws(T, d, E, dtype) : 0;
    const size_t need = front + forward_ws(T, d, E, K, n, dtype, st);
    if (ws == nullptr || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "%s needs %zu workspace bytes (got %zu)", name, need, ws_bytes);
    if (!aligned16(ws)) return fail(MOE_ERR_INVALID_ARG, "ws must be 16-byte aligned");

    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t A = (size_t)T * K;
    const size_t sz = elem_bytes(dtype);
    const int B = count_rows(T, st);
    Carver c(ws);
    void* front_ws = c.take<char>(front);
    int32_t* blk = c.take<int32_t>((size_t)B * E);
    int32_t* blkbase = c.take<int32_t>((size_t)B * E);
    int32_t* ws_idx = c.take<int32_t>(A);
    float* ws_w = c.take<float>(A);
    int32_t* ws_cnt = c.take<int32_t>(E);
    int32_t* ws_off = c.take<int32_t>(E + 1);
    int32_t* ws_sp = c.take<int32_t>(A);
    int32_t* ws_inv = c.take<int32_t>(A);
    const bool gather = ffn_gather_ok(dtype, T, d, n);
    void* Xp = gather ? nullptr : c.take<char>(A * d * sz);
    void* Yb = c.take<char>(A * d * sz);
    void* Act = c.take<char>(A * n * sz);
    const size_t split_bytes = ffn_split_bytes(dtype, d, n);
    float* part = split_bytes ? c.take<float>(split_bytes / sizeof(float)) : nullptr;
    if (!topk_idx) topk_idx = ws_idx;
    if (!topk_w) topk_w = ws_w;
    if (!counts) counts = ws_cnt;
    if (!offsets) offsets = ws_off;
    if (!sorted_pair) sorted_pair = ws_sp;
    if (!inv) inv = ws_inv;

    if (from_x) CHECK(route_x_front(X, dtype, T, d, E, K, Wr, bias, logits_out, topk_idx, topk_w, blk, front_ws, s));
    else HIPCHECK(launch_gate(logits_in, T, E, K, topk_idx, topk_w, blk, s));
    // the scan also clears the grouped GEMMs' claim counters (no launches of their own)
    int* tickets = ffn_tickets(part);
    const int nt = tickets != nullptr ? ffn_ticket_ints() : 0;
    if (scan_rank_fused(T, E, st)) {
        HIPCHECK(launch_scan_rank(topk_idx, T, E, K, blk, counts, offsets, sorted_pair, inv, tickets, nt, s, st));
    } else {
        HIPCHECK(launch_scan(blk, B, E, counts, offsets, blkbase, s, tickets, nt));
        HIPCHECK(launch_rank(topk_idx, T, E, K, blkbase, sorted_pair, inv, s, st));
    }
    if (gather) {
        // no permuted copy of X: the SwiGLU GEMM gathers its rows through sorted_pair
        HIPCHECK(launch_ffn(X, W1, W3, W2, dtype, (int)A, d, E, n, counts, offsets, Act, Yb, part, true, s,
                            sorted_pair, K, T));
    } else {
        HIPCHECK(launch_copy_rows(X, (size_t)d * sz, T, K, inv, Xp, s));
        HIPCHECK(launch_ffn(Xp, W1, W3, W2, dtype, (int)A, d, E, n, counts, offsets, Act, Yb, part, true, s));
    }
    HIPCHECK(launch_combine(Yb, topk_w, inv, dtype, T, d, K, out, s));
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward(const void* X, const float* logits, const void* W1, const void* W3, const void* W2,
                int dtype, int T, int d, int E, int K, int n, void* out, int32_t* topk_idx,
                float* topk_w, int32_t* counts, int32_t* offsets, int32_t* sorted_pair, int32_t* inv,
                void* ws, size_t ws_bytes, void* stream) {
    return forward_impl("moe_forward", X, logits, nullptr, nullptr, nullptr, W1, W3, W2, dtype, T, d, E, K, n, out,
                        topk_idx, topk_w, counts, offsets, sorted_pair, inv, ws, ws_bytes, stream);
}

int moe_route_x(const void* X, int dtype, int T, int d, int E, int K, const float* Wr, const float* bias,
                float* logits, int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets, void* ws,
                size_t ws_bytes, void* stream) {
    CHECK(check_tek(T, E, K));
    CHECK(check_router(T, d, E));
    CHECK(check_dtype(dtype));
    NONNULL(X);
    NONNULL(Wr);
    NONNULL(topk_idx);
    NONNULL(topk_w);
    NONNULL(counts);
    NONNULL(offsets);
    for (const void* p : {(const void*)logits, (const void*)bias})
        if (p != nullptr && !aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "logits and bias must be 16-byte aligned");
    const int st = route_x_rows_tokens(dtype, d, E);
    const size_t front = route_x_front_ws(T, d, E, dtype);
    const size_t need = front + align_up((size_t)count_rows(T, st) * E * sizeof(int32_t));
    if (ws == nullptr || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "moe_route_x needs %zu workspace bytes (got %zu)", need, ws_bytes);
    if (!aligned16(ws)) return fail(MOE_ERR_INVALID_ARG, "ws must be 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    Carver c(ws);
    void* front_ws = c.take<char>(front);
    int32_t* blk = c.take<int32_t>((size_t)count_rows(T, st) * E);
    CHECK(route_x_front(X, dtype, T, d, E, K, Wr, bias, logits, topk_idx, topk_w, blk, front_ws, s));
    HIPCHECK(launch_scan(blk, count_rows(T, st), E, counts, offsets, nullptr, s));
    return MOE_OK;
}

int moe_forward_x(const void* X, const float* Wr, const float* bias, const void* W1, const void* W3, const void* W2,
                  int dtype, int T, int d, int E, int K, int n, void* out, float* logits, int32_t* topk_idx,
                  float* topk_w, int32_t* counts, int32_t* offsets, int32_t* sorted_pair, int32_t* inv, void* ws,
                  size_t ws_bytes, void* stream) {
    if (Wr == nullptr) return fail(MOE_ERR_INVALID_ARG, "Wr must not be NULL");
    return forward_impl("moe_forward_x", X, nullptr, Wr, bias, logits, W1, W3, W2, dtype, T, d, E, K, n, out,
                        topk_idx, topk_w, counts, offsets, sorted_pair, inv, ws, ws_bytes, stream);
}

long long moe_token_round_max_rows(int T, int E, int K, int M) {
    if (check_tr(T, E, K, M, 0) != MOE_OK) return 0;
    return tr_max_rows(T, E, K, M);
}

size_t moe_token_round_workspace_bytes(int T, int E, int K, int M) {
    if (check_tr(T, E, K, M, 0) != MOE_OK) return 0;
    return align_up(tr_keys_bytes(T, E));
}

int moe_token_round(const float* logits, const int32_t* topk_idx, const int32_t* counts, int T, int E, int K,
                    int M, int cap_tiles, int32_t* counts_r, int32_t* offsets_r, int32_t* row_tok,
                    long long rows_cap, int32_t* slot_row, float* slot_w, void* ws, size_t ws_bytes,
                    void* stream) {
    CHECK(check_tr(T, E, K, M, cap_tiles));
    NONNULL(logits);
    NONNULL(topk_idx);
    NONNULL(counts);
    NONNULL(counts_r);
    NONNULL(offsets_r);
    NONNULL(row_tok);
    NONNULL(slot_row);
    NONNULL(slot_w);
    const long long need_rows = tr_max_rows(T, E, K, M);
    if (rows_cap < need_rows)
        return fail(MOE_ERR_INVALID_ARG, "row_tok needs room for %lld rows (got %lld)", need_rows, rows_cap);
    const size_t need = align_up(tr_keys_bytes(T, E));
    if (ws == nullptr || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "moe_token_round needs %zu workspace bytes (got %zu)", need, ws_bytes);
    if (!aligned16(ws)) return fail(MOE_ERR_INVALID_ARG, "ws must be 16-byte aligned");
    HIPCHECK(launch_token_round(logits, topk_idx, counts, T, E, K, M, cap_tiles, counts_r, offsets_r, row_tok,
                                need_rows, slot_row, slot_w, ws, static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

int moe_tr_combine(const void* Y, const int32_t* slot_row, const float* slot_w, int dtype, int T, int E, int d,
                   long long rows, void* out, void* stream) {
    if (T < 1) return fail(MOE_ERR_INVALID_ARG, "T must be >= 1 (got %d)", T);
    if (E < 1) return fail(MOE_ERR_INVALID_ARG, "E must be >= 1 (got %d)", E);
    if (E > kMaxE) return fail(MOE_ERR_UNSUPPORTED, "E=%d exceeds the supported maximum %d", E, kMaxE);
    if ((long long)T * E >= (1LL << 31)) return fail(MOE_ERR_UNSUPPORTED, "T*E must be < 2^31");
    if (rows < 0 || rows >= (1LL << 31)) return fail(MOE_ERR_INVALID_ARG, "rows must be in [0, 2^31)");
    CHECK(check_dtype(dtype));
    CHECK(check_row(d, dtype));
    NONNULL(Y);
    NONNULL(slot_row);
    NONNULL(slot_w);
    NONNULL(out);
    HIPCHECK(launch_tr_combine(Y, slot_row, slot_w, dtype, T, E, d, rows, out, static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

size_t moe_forward_tr_workspace_bytes(int T, int d, int E, int K, int n, int M, int dtype) {
    if (check_tr(T, E, K, M, 0) != MOE_OK || check_dtype(dtype) != MOE_OK || check_dim("d", d, dtype) != MOE_OK ||
        check_dim("n", n, dtype) != MOE_OK)
        return 0;
    return forward_tr_ws(T, d, E, K, n, M, dtype);
}

int moe_forward_tr(const void* X, const float* logits, const void* W1, const void* W3, const void* W2, int dtype,
                   int T, int d, int E, int K, int n, int M, int cap_tiles, void* out, int32_t* counts_r,
                   int32_t* offsets_r, int32_t* row_tok, int32_t* slot_row, float* slot_w, void* ws,
                   size_t ws_bytes, void* stream) {
    CHECK(check_tr(T, E, K, M, cap_tiles));
    CHECK(check_dtype(dtype));
    CHECK(check_dim("d", d, dtype));
    CHECK(check_dim("n", n, dtype));
    NONNULL(X);
    NONNULL(logits);
    NONNULL(W1);
    NONNULL(W3);
    NONNULL(W2);
    NONNULL(out);
    for (const void* p : {(const void*)counts_r, (const void*)offsets_r, (const void*)row_tok,
                          (const void*)slot_row, (const void*)slot_w})
        if (p != nullptr && !aligned16(p))
            return fail(MOE_ERR_INVALID_ARG, "optional outputs must be 16-byte aligned");
    const long long R = tr_max_rows(T, E, K, M);
    if (R >= (1LL << 31)) return fail(MOE_ERR_UNSUPPORTED, "the plan's row bound must be < 2^31");
    if (R * (long long)(d > n ? d : n) >= (1LL << 40))
        return fail(MOE_ERR_UNSUPPORTED, "rows*max(d,n) must be < 2^40");
    const size_t need = forward_tr_ws(T, d, E, K, n, M, dtype);
    if (ws == nullptr || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "moe_forward_tr needs %zu workspace bytes (got %zu)", need, ws_bytes);
    if (!aligned16(ws)) return fail(MOE_ERR_INVALID_ARG, "ws must be 16-byte aligned");

    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t A = (size_t)T * K;
    const size_t sz = elem_bytes(dtype);
    const int B = num_chunks(T);
    const bool gather = ffn_gather_ok(dtype, T, d, n);
    Carver c(ws);
    int32_t* blk = c.take<int32_t>((size_t)B * E);
    int32_t* blkbase = c.take<int32_t>((size_t)B * E);
    int32_t* idx = c.take<int32_t>(A);
    float* w = c.take<float>(A);
    int32_t* counts = c.take<int32_t>(E);
    int32_t* offsets = c.take<int32_t>(E + 1);
    void* keys = c.take<char>(tr_keys_bytes(T, E));
    int32_t* ws_cr = c.take<int32_t>(E);
    int32_t* ws_or = c.take<int32_t>(E + 1);
    int32_t* ws_rt = c.take<int32_t>((size_t)R);
    int32_t* ws_sr = c.take<int32_t>((size_t)T * E);
    float* ws_sw = c.take<float>((size_t)T * E);
    void* Xp = gather ? nullptr : c.take<char>((size_t)R * d * sz);
    void* Yb = c.take<char>((size_t)R * d * sz);
    void* Act = c.take<char>((size_t)R * n * sz);
    const size_t split_bytes = ffn_split_bytes(dtype, d, n);
    float* part = split_bytes ? c.take<float>(split_bytes / sizeof(float)) : nullptr;
    if (!counts_r) counts_r = ws_cr;
    if (!offsets_r) offsets_r = ws_or;
    if (!row_tok) row_tok = ws_rt;
    if (!slot_row) slot_row = ws_sr;
    if (!slot_w) slot_w = ws_sw;

    HIPCHECK(launch_gate(logits, T, E, K, idx, w, blk, s));
    // the scan also clears the grouped GEMMs' claim counters
    int* tickets = ffn_tickets(part);
    HIPCHECK(launch_scan(blk, B, E, counts, offsets, blkbase, s, tickets, tickets != nullptr ? ffn_ticket_ints() : 0));
    HIPCHECK(launch_token_round(logits, idx, counts, T, E, K, M, cap_tiles, counts_r, offsets_r, row_tok, R, slot_row,
                                slot_w, keys, s));
    if (gather) {
        HIPCHECK(launch_ffn(X, W1, W3, W2, dtype, (int)R, d, E, n, counts_r, offsets_r, Act, Yb, part, true, s,
                            row_tok, 1, T));
    } else {
        HIPCHECK(launch_tr_gather_rows(X, (size_t)d * sz, T, row_tok, offsets_r, E, R, Xp, s));
        HIPCHECK(launch_ffn(Xp, W1, W3, W2, dtype, (int)R, d, E, n, counts_r, offsets_r, Act, Yb, part, true, s));
    }
    HIPCHECK(launch_tr_combine(Yb, slot_row, slot_w, dtype, T, E, d, R, out, s));
    return MOE_OK;
}

size_t moe_backward_data_workspace_bytes(int T, int d, int E, int K, int n, int dtype) {
    if (check_tek(T, E, K) != MOE_OK || check_dtype(dtype) != MOE_OK || check_dim("d", d, dtype) != MOE_OK ||
        check_dim("n", n, dtype) != MOE_OK)
        return 0;
    return backward_ws(T, d, E, K, n, dtype, false);
}

size_t moe_backward_workspace_bytes(int T, int d, int E, int K, int n, int dtype) {
    if (check_tek(T, E, K) != MOE_OK || check_dtype(dtype) != MOE_OK || check_dim("d", d, dtype) != MOE_OK ||
        check_dim("n", n, dtype) != MOE_OK)
        return 0;
    return backward_ws(T, d, E, K, n, dtype, true);
}

}  // extern "C"

namespace {

// The backward of both entry points; the weight gradients when dW1 is not NULL.
int backward_impl(const char* name, const void* X, const float* logits, const void* W1, const void* W3,
                  const void* W2, int dtype, int T, int d, int E, int K, int n, const void* dout, void* dX,
                  float* dlogits, float* dw, float* dW1, float* dW3, float* dW2, void* ws, size_t ws_bytes,
                  void* stream) {
    CHECK(check_tek(T, E, K));
    CHECK(check_dtype(dtype));
    CHECK(check_dim("d", d, dtype));
    CHECK(check_dim("n", n, dtype));
    NONNULL(X);
    NONNULL(logits);
    NONNULL(W1);
    NONNULL(W3);
    NONNULL(W2);
    NONNULL(dout);
    NONNULL(dX);
    NONNULL(dlogits);
    const bool weights = dW1 != nullptr;
    if (weights) {
        NONNULL(dW3);
        NONNULL(dW2);
    }
    if (dw != nullptr && !aligned16(dw)) return fail(MOE_ERR_INVALID_ARG, "dw must be 16-byte aligned");
    if ((long long)T * K * 2LL * (long long)(d > n ? d : n) >= (1LL << 40))
        return fail(MOE_ERR_UNSUPPORTED, "T*K*2*max(d,n) must be < 2^40");
    const size_t need = backward_ws(T, d, E, K, n, dtype, weights);
    if (ws == nullptr || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "%s needs %zu workspace bytes (got %zu)", name, need, ws_bytes);
    if (!aligned16(ws)) return fail(MOE_ERR_INVALID_ARG, "ws must be 16-byte aligned");

    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t A = (size_t)T * K;
    const size_t sz = elem_bytes(dtype);
    const int B = num_chunks(T);
    Carver c(ws);
    int32_t* blk = c.take<int32_t>((size_t)B * E);
    int32_t* blkbase = c.take<int32_t>((size_t)B * E);
    int32_t* idx = c.take<int32_t>(A);
    float* w = c.take<float>(A);
    int32_t* counts = c.take<int32_t>(E);
    int32_t* offsets = c.take<int32_t>(E + 1);
    int32_t* sorted_pair = c.take<int32_t>(A);
    int32_t* inv = c.take<int32_t>(A);
    float* ws_ds = c.take<float>(A);
    float* ones = c.take<float>(A);
    void* Xp = c.take<char>(A * d * sz);  // later dXp
    void* dY = c.take<char>(A * d * sz);
    void* H1 = c.take<char>(2 * A * n * sz);  // H1, then H3
    void* H3 = static_cast<char*>(H1) + A * n * sz;
    void* dA = c.take<char>(A * n * sz);
    void* dH = c.take<char>(A * 2 * n * sz);
    // The bf16 pipelined GEMM reads W2 and W1, W3 k-contiguous as they are;
    // the other kernels multiply by transposed copies.
    const bool bt_da = ffn_bt_ok(dtype, n, d, d), bt_dx = ffn_bt_ok(dtype, d, 2 * n, n);
    void* W2t = bt_da ? nullptr : c.take<char>((size_t)E * d * n * sz);
    void* W13t = bt_dx ? nullptr : c.take<char>((size_t)E * 2 * d * n * sz);
    const size_t split_bytes = ffn_split_bytes(dtype, 256, 128);
    float* part = split_bytes ? c.take<float>(split_bytes / sizeof(float)) : nullptr;
    void* aw = weights ? c.take<char>(A * n * sz) : nullptr;
    float* dS = dw != nullptr ? dw : ws_ds;

    // routing, as in moe_forward
    HIPCHECK(launch_gate(logits, T, E, K, idx, w, blk, s));
    if (scan_rank_fused(T, E)) {
        HIPCHECK(launch_scan_rank(idx, T, E, K, blk, counts, offsets, sorted_pair, inv, nullptr, 0, s));
    } else {
        HIPCHECK(launch_scan(blk, B, E, counts, offsets, blkbase, s));
        HIPCHECK(launch_rank(idx, T, E, K, blkbase, sorted_pair, inv, s));
    }
    // expert-sorted rows of X and of dout
    HIPCHECK(launch_copy_rows(X, (size_t)d * sz, T, K, inv, Xp, s));
    HIPCHECK(launch_copy_rows(dout, (size_t)d * sz, T, K, inv, dY, s));
    // transposed weights where needed: W2^T [E, d, n]; [W1^T ; W3^T] [E, 2n, d]
    if (!bt_da) HIPCHECK(launch_transpose_experts(W2, dtype, E, n, d, W2t, (size_t)d * n, (size_t)n, s));
    if (!bt_dx) {
        HIPCHECK(launch_transpose_experts(W1, dtype, E, d, n, W13t, (size_t)2 * n * d, (size_t)d, s));
        HIPCHECK(launch_transpose_experts(W3, dtype, E, d, n, static_cast<char*>(W13t) + (size_t)n * d * sz,
                                          (size_t)2 * n * d, (size_t)d, s));
    }
    // pre-activations H1 = Xp W1, H3 = Xp W3; dA = dY W2^T (grouped, per expert)
    if (ffn_raw_ok(dtype, d, n)) {
        // one launch of the SwiGLU GEMM's kernel, storing both pre-activations
        HIPCHECK(launch_ffn_up_raw(Xp, W1, W3, (int)A, d, E, n, counts, offsets, H1, s));
    } else {
        HIPCHECK(launch_ffn_down(Xp, W1, dtype, (int)A, n, E, d, counts, offsets, H1, part, false, s));
        HIPCHECK(launch_ffn_down(Xp, W3, dtype, (int)A, n, E, d, counts, offsets, H3, part, false, s));
    }
    if (bt_da) {
        // dA = dY W2^T with the SwiGLU backward and dS in the GEMM's epilogue
        // (dA is never stored; its buffer holds the row weights and dS parts)
        float* wrow = static_cast<float*>(dA);
        float* ds_part = wrow + align_up(A * sizeof(float)) / sizeof(float);
        HIPCHECK(launch_row_weights(w, sorted_pair, (int)A, wrow, s));
        HIPCHECK(launch_ffn_bt_swiglu_bwd(dY, W2, d, (int)A, n, E, counts, offsets, H1, H3, dH, aw, wrow, ds_part, s));
        HIPCHECK(launch_ds_reduce(ds_part, n / 64, sorted_pair, (int)A, dS, s));
    } else {
        HIPCHECK(launch_ffn_down(dY, W2t, dtype, (int)A, n, E, d, counts, offsets, dA, part, false, s));
        // SwiGLU backward and dS (and w * act for dW2)
        HIPCHECK(launch_swiglu_bwd(H1, H3, dA, w, sorted_pair, dtype, (int)A, n, dH, dS, aw, s));
    }
    if (weights) {
        // dW1 = Xp^T dh1, dW3 = Xp^T dh3, dW2 = (w act)^T dY, over each expert's rows
        HIPCHECK(launch_dw(Xp, d, dH, 2 * n, 0, counts, offsets, dtype, E, d, n, (int)A, dW1, s));
        HIPCHECK(launch_dw(Xp, d, dH, 2 * n, n, counts, offsets, dtype, E, d, n, (int)A, dW3, s));
        HIPCHECK(launch_dw(aw, n, dY, d, 0, counts, offsets, dtype, E, n, d, (int)A, dW2, s));
    }
    // dXp = [dh1 | dh3] [W1^T ; W3^T] (overwrites Xp)
    if (bt_dx) HIPCHECK(launch_ffn_bt(dH, W1, W3, n, dtype, (int)A, d, E, 2 * n, counts, offsets, Xp, part, false, s));
    else HIPCHECK(launch_ffn_down(dH, W13t, dtype, (int)A, d, E, 2 * n, counts, offsets, Xp, part, false, s));
    // dX[t] = sum over the token's rows, unit weights; logit gradient from dS
    HIPCHECK(launch_fill_f32(ones, A, 1.0f, s));
    HIPCHECK(launch_combine(Xp, ones, inv, dtype, T, d, K, dX, s));
    HIPCHECK(launch_logit_grad(idx, w, dS, T, E, K, dlogits, s));
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_backward_data(const void* X, const float* logits, const void* W1, const void* W3, const void* W2, int dtype,
                      int T, int d, int E, int K, int n, const void* dout, void* dX, float* dlogits, float* dw,
                      void* ws, size_t ws_bytes, void* stream) {
    return backward_impl("moe_backward_data", X, logits, W1, W3, W2, dtype, T, d, E, K, n, dout, dX, dlogits, dw,
                         nullptr, nullptr, nullptr, ws, ws_bytes, stream);
}

int moe_backward(const void* X, const float* logits, const void* W1, const void* W3, const void* W2, int dtype, int T,
                 int d, int E, int K, int n, const void* dout, void* dX, float* dlogits, float* dw, float* dW1,
                 float* dW3, float* dW2, void* ws, size_t ws_bytes, void* stream) {
    if (dW1 == nullptr) return fail(MOE_ERR_INVALID_ARG, "dW1 must not be NULL");
    return backward_impl("moe_backward", X, logits, W1, W3, W2, dtype, T, d, E, K, n, dout, dX, dlogits, dw, dW1,
                         dW3, dW2, ws, ws_bytes, stream);
}

}  // extern "C"
