// mhla_api.hip -- the C ABI declared in include/mhla.h.
//
// Host-side only: argument validation (before anything is enqueued), the
// stream-ordered workspace for the two summary arrays, and the sequence
// summaries -> mixing -> output on the caller's stream.  No call synchronises
// the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "common.hpp"
#include "kernels.hpp"
#include "mhla.h"

namespace mhla {

int device_cu_count() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices];  // 0: not queried yet (static storage starts zeroed)
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 256;
    }
    if (dev >= 0 && dev < kMaxDevices) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) {
        (void)hipGetLastError();
        cus = 256;
    }
    if (dev >= 0 && dev < kMaxDevices) cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

}  // namespace mhla

namespace {

thread_local char g_err[512] = "";

// Test hook (mhla_debug_fail_workspace): number of upcoming workspace requests that
// fail as if the allocation had failed.
std::atomic<int> g_fail_workspace{0};

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_err[0] = '\0';
    return MHLA_OK;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(MHLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_ptr(const void* p, const char* name) {
    if (!p) return fail(MHLA_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned16(p)) return fail(MHLA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
    return MHLA_OK;
}

// Sizes shared by every entry point.  Element counts must fit in int64 with
// margin, and grid sizes in 32 bits.
int check_sizes(int64_t B, int64_t H, int64_t N, int64_t d, int64_t M, bool equal_blocks = true) {
    if (B < 1 || H < 1 || N < 1 || d < 1 || M < 1)
        return fail(MHLA_ERR_INVALID_ARG, "sizes must be >= 1 (B=%lld H=%lld N=%lld d=%lld M=%lld)",
                    (long long)B, (long long)H, (long long)N, (long long)d, (long long)M);
    if (equal_blocks && N % M != 0)
        return fail(MHLA_ERR_INVALID_ARG, "N=%lld is not a multiple of M=%lld", (long long)N, (long long)M);
    if (d != 16 && d != 32 && d != 64)
        return fail(MHLA_ERR_UNSUPPORTED, "d=%lld is not one of 16, 32, 64", (long long)d);
    const int64_t lim = (int64_t)1 << 40;
    if (B > lim / H || B * H > lim / N || B * H * N > lim / d)
        return fail(MHLA_ERR_INVALID_ARG, "tensor too large");
    if (N * d > ((int64_t)1 << 30))  // kernels index inside one (batch, head) pair with 32-bit offsets
        return fail(MHLA_ERR_UNSUPPORTED, "N*d=%lld exceeds 2^30", (long long)(N * d));
    if (M > 65536 || B * H * M > ((int64_t)1 << 29))
        return fail(MHLA_ERR_UNSUPPORTED, "too many blocks (M=%lld, B*H*M=%lld)", (long long)M,
                    (long long)(B * H * M));
    return MHLA_OK;
}

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

int64_t summary_floats(int64_t d) { return d * d + d; }

// One memory pool per device for the forward-pass workspace.  Its release
// threshold keeps freed blocks for reuse, so steady-state calls do not go back
// to the driver.
struct Pools {
    std::mutex mu;
    std::vector<hipMemPool_t> pools;
    std::vector<bool> made;
};
Pools& pools() {
    static Pools p;
    return p;
}

hipError_t device_pool(hipMemPool_t* out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    Pools& P = pools();
    std::lock_guard<std::mutex> lock(P.mu);
    if ((int)P.pools.size() <= dev) {
        P.pools.resize(dev + 1, nullptr);
        P.made.resize(dev + 1, false);
    }
    if (!P.made[dev]) {
        hipMemPoolProps props;
        memset(&props, 0, sizeof props);
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        e = hipMemPoolCreate(&pool, &props);
        if (e != hipSuccess) return e;
        uint64_t keep = UINT64_MAX;
        e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
        if (e != hipSuccess) return e;
        P.pools[dev] = pool;
        P.made[dev] = true;
    }
    *out = P.pools[dev];
    return hipSuccess;
}

// Two summary arrays (S, St), the mixing kernel's split-W fragments, then the
// summary kernel's partial sums when it cuts long blocks into token segments.
// nw: number of M x M mixing matrices (H with one per head, else 1).
size_t frag_bytes_aligned(int64_t M, int64_t nw = 1) {
    return (nw * mhla::mix_fragment_bytes(M) + 255) / 256 * 256;
}

// cmax: the longest block (N / M for equal blocks).
size_t workspace_bytes(int dtype, int64_t BH, int64_t cmax, int64_t d, int64_t M, int64_t nw = 1) {
    return 2 * (size_t)(M * BH * summary_floats(d)) * sizeof(float) + frag_bytes_aligned(M, nw) +
           mhla::summary_partial_bytes(dtype, BH, cmax, (int)d, M);
}

int pool_alloc(void** ptr, size_t bytes, hipStream_t stream) {
    hipMemPool_t pool = nullptr;
    hipError_t e = device_pool(&pool);
    if (e != hipSuccess) return hip_fail(e, "workspace pool");
    *ptr = nullptr;
    e = hipMallocFromPoolAsync(ptr, bytes, pool, stream);
    if (e != hipSuccess || !*ptr) {
        (void)hipGetLastError();
        return fail(MHLA_ERR_NO_MEMORY, "workspace of %zu bytes: %s", bytes, hipGetErrorString(e));
    }
    return MHLA_OK;
}

// Workspace kept per (device, stream).  Calls on one stream run in order, so they can
// share one buffer; a steady-state call then makes no allocation call at all (a
// stream-ordered malloc/free pair per call made the host wait for the GPU on every
// call on this runtime).  A call that needs more takes a larger buffer from the pool
// (at least 1.5x the old one) and frees the old one in stream order.  Calls on
// different streams use different buffers.
//
// A call made while its stream is being captured into a graph must not use that
// buffer: memory allocated during capture belongs to the graph (it is not valid once
// the graph is gone), and a graph replayed later could overlap eager calls on the
// stream.  Such a call allocates its own workspace from the pool and frees it at its
// end, both in stream order, so the graph holds an allocation and a free node of its
// own (*owned = true: the caller frees it).
struct StreamWorkspace {
    int dev;
    hipStream_t stream;
    void* ptr;
    size_t bytes;
};
struct WorkspaceCache {
    std::mutex mu;
    std::vector<StreamWorkspace> live;
};
WorkspaceCache& workspace_cache() {
    static WorkspaceCache c;
    return c;
}

int stream_workspace(size_t bytes, hipStream_t stream, void** out, bool* owned) {
    *out = nullptr;
    *owned = false;
    if (bytes == 0) return MHLA_OK;
    for (int n = g_fail_workspace.load(); n > 0;)
        if (g_fail_workspace.compare_exchange_weak(n, n - 1))
            return fail(MHLA_ERR_NO_MEMORY, "workspace of %zu bytes: allocation failure simulated by the test hook",
                        bytes);
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
        (void)hipGetLastError();
        cs = hipStreamCaptureStatusNone;
    }
    if (cs != hipStreamCaptureStatusNone) {
        const int st = pool_alloc(out, bytes, stream);
        if (st) return st;
        *owned = true;
        return MHLA_OK;
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "workspace device");
    WorkspaceCache& c = workspace_cache();
    std::lock_guard<std::mutex> lock(c.mu);
    StreamWorkspace* entry = nullptr;
    for (auto& w : c.live)
        if (w.dev == dev && w.stream == stream) entry = &w;
    if (entry && entry->bytes >= bytes) {
        *out = entry->ptr;
        return MHLA_OK;
    }
    size_t want = entry ? std::max(bytes, entry->bytes + entry->bytes / 2) : bytes;
    want = (want + (2u << 20) - 1) / (2u << 20) * (2u << 20);
    void* p = nullptr;
    const int st = pool_alloc(&p, want, stream);
    if (st) return st;
    if (entry) {
        e = hipFreeAsync(entry->ptr, stream);  // after the calls already enqueued that use it
        if (e != hipSuccess) {
            (void)hipFreeAsync(p, stream);
            return hip_fail(e, "workspace release");
        }
        entry->ptr = p;
        entry->bytes = want;
    } else {
        c.live.push_back({dev, stream, p, want});
    }
    *out = p;
    return MHLA_OK;
}

// Releases a workspace that stream_workspace() handed to this call alone.
hipError_t release_workspace(void* ws, bool owned, hipStream_t stream) {
    return owned && ws ? hipFreeAsync(ws, stream) : hipSuccess;
}

// Scratch memory of mhla_forward_noalloc: a file-scope device array, one copy per device
// (each holds it from the moment the library's code is loaded there until the process
// ends).  In host code `scratch` names a host-side stand-in, not device memory: the
// device address of each device's copy is looked up once, with that device current,
// and only that address is used.
constexpr size_t kNoAllocScratchBytes = size_t(MHLA_NOALLOC_SCRATCH_BYTES);
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

struct ScratchAddresses {
    std::mutex mu;
    std::vector<void*> ptr;  // per device; null until looked up
};
ScratchAddresses& scratch_addresses() {
    static ScratchAddresses a;
    return a;
}

int fixed_workspace(void** out) {
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "scratch device");
    ScratchAddresses& a = scratch_addresses();
    std::lock_guard<std::mutex> lock(a.mu);
    if ((int)a.ptr.size() <= dev) a.ptr.resize(dev + 1, nullptr);
    if (!a.ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "scratch array address");
        }
        a.ptr[dev] = p;
    }
    *out = a.ptr[dev];
    return MHLA_OK;
}

// Frees the cached workspace of (current device, stream), in stream order.
int drop_stream_workspace(hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "workspace device");
    WorkspaceCache& c = workspace_cache();
    std::lock_guard<std::mutex> lock(c.mu);
    for (size_t i = 0; i < c.live.size(); ++i) {
        if (c.live[i].dev != dev || c.live[i].stream != stream) continue;
        e = hipFreeAsync(c.live[i].ptr, stream);  // after the work already enqueued that uses it
        if (e != hipSuccess) return hip_fail(e, "workspace release");
        c.live.erase(c.live.begin() + (std::ptrdiff_t)i);
        break;
    }
    return ok();
}

int forward_path(int64_t B, int64_t H, int64_t N, int64_t d, int64_t M, int causal, int dtype) {
    if (dtype != mhla::kDtypeBF16 || causal) return MHLA_PATH_STAGED;
    if (mhla::fused_applicable((int)d, B * H, N, M)) return MHLA_PATH_FUSED;
    if (mhla::pair_applicable((int)d, B * H, N, M)) return MHLA_PATH_PAIR;
    return MHLA_PATH_STAGED;
}

constexpr unsigned kKnownOptions = MHLA_OPT_CAUSAL | MHLA_OPT_NO_NORMALIZER | MHLA_OPT_OUT_BF16 | MHLA_OPT_W_PER_HEAD;

// order/offsets: a token list per block (both null: M equal contiguous blocks);
// max_block bounds the block lengths for launch planning.
// fixed: when given, the staged path takes its workspace from there (at most
// fixed_cap bytes; larger needs give MHLA_ERR_UNSUPPORTED before anything is enqueued)
// instead of the stream's cached workspace, so the call allocates nothing.
int fixed_workspace(void** out);

int forward_impl(int dtype, const void* q, const void* k, const void* v, const float* W, void* out, int64_t B,
                 int64_t H, int64_t N, int64_t d, int64_t M, unsigned options, const int32_t* order,
                 const int32_t* offsets, int64_t max_block, mhla_stream_t stream_, bool fixed = false,
                 size_t fixed_cap = 0) {
    const bool listed = order || offsets;
    int st = check_sizes(B, H, N, d, M, !listed);
    if (st) return st;
    if (options & ~kKnownOptions) return fail(MHLA_ERR_INVALID_ARG, "unknown option bits 0x%x", options & ~kKnownOptions);
    if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
        (st = check_ptr(W, "W")) || (st = check_ptr(out, "out")))
        return st;
    const int causal = (options & MHLA_OPT_CAUSAL) != 0;
    if (listed) {
        if (!order || !offsets) return fail(MHLA_ERR_INVALID_ARG, "order and offsets must both be given");
        if (((uintptr_t)order & 3u) || ((uintptr_t)offsets & 3u))
            return fail(MHLA_ERR_INVALID_ARG, "order and offsets must be 4-byte aligned");
        if (max_block < 1 || max_block > N)
            return fail(MHLA_ERR_INVALID_ARG, "max_block=%lld is outside [1, N]", (long long)max_block);
        if (causal) return fail(MHLA_ERR_UNSUPPORTED, "token-list blocks are non-causal only");
    } else {
        max_block = N / M;
    }
    const mhla::BlockLayout lay{order, offsets};
    const mhla::OutSpec os{out, (options & MHLA_OPT_OUT_BF16) != 0, (options & MHLA_OPT_NO_NORMALIZER) == 0};
    const int heads = (options & MHLA_OPT_W_PER_HEAD) ? (int)H : 0;  // H fits: B*H*M <= 2^29
    const int64_t nw = heads ? H : 1;
    const size_t esz = dtype == mhla::kDtypeF32 ? 4 : 2;
    const size_t in_bytes = (size_t)(B * H * N * d) * esz;
    const size_t out_bytes = (size_t)(B * H * N * d) * (os.bf16 ? 2 : 4);
    if (overlaps(out, out_bytes, q, in_bytes) || overlaps(out, out_bytes, k, in_bytes) ||
        overlaps(out, out_bytes, v, in_bytes) || overlaps(out, out_bytes, W, (size_t)(nw * M * M) * 4))
        return fail(MHLA_ERR_INVALID_ARG, "out overlaps an input");

    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    const int64_t BH = B * H;
    const int path = listed ? MHLA_PATH_STAGED : forward_path(B, H, N, d, M, causal, dtype);
    if (path == MHLA_PATH_FUSED) {
        hipError_t e = mhla::launch_fused(q, k, v, W, os, BH, N, (int)d, M, heads, stream);
        if (e != hipSuccess) return hip_fail(e, "fused kernel");
        return ok();
    }
    if (path == MHLA_PATH_PAIR) {
        hipError_t e = mhla::launch_pair(q, k, v, W, os, BH, N, (int)d, M, heads, stream);
        if (e != hipSuccess) return hip_fail(e, "pair kernel");
        return ok();
    }
    const size_t arr = (size_t)(M * BH * summary_floats(d)) * sizeof(float);
    const size_t total = workspace_bytes(dtype, BH, max_block, d, M, nw);
    void* ws = nullptr;
    bool owned = false;
    if (fixed) {
        if (total > fixed_cap)
            return fail(MHLA_ERR_UNSUPPORTED, "these sizes need %zu bytes of workspace, more than the %zu-byte scratch "
                        "array of the non-allocating entry point", total, fixed_cap);
        const int st2 = fixed_workspace(&ws);
        if (st2) return st2;
    } else {
        const int st2 = stream_workspace(total, stream, &ws, &owned);
        if (st2) return st2;
    }
    float* S = static_cast<float*>(ws);
    float* St = S + arr / sizeof(float);
    void* frags = St + arr / sizeof(float);
    float* partial = mhla::summary_partial_bytes(dtype, BH, max_block, (int)d, M)
                         ? reinterpret_cast<float*>(static_cast<char*>(frags) + frag_bytes_aligned(M, nw))
                         : nullptr;
    const char* what = "summary kernel";
    hipError_t e = mhla::launch_summaries(dtype, k, v, S, BH, N, (int)d, M, heads, lay, max_block, partial, stream);
    if (e == hipSuccess) {
        what = "mixing kernel";
        e = mhla::launch_mix(S, W, St, BH, (int)d, M, causal != 0, dtype == mhla::kDtypeF32, heads, frags, stream);
    }
    if (e == hipSuccess) {
        what = "output kernel";
        e = mhla::launch_output(dtype, q, k, v, St, W, os, BH, N, (int)d, M, causal != 0, heads, lay, max_block,
                                stream);
    }
    const hipError_t fe = release_workspace(ws, owned, stream);
    if (e != hipSuccess) return hip_fail(e, what);
    if (fe != hipSuccess) return hip_fail(fe, "workspace release");
    return ok();
}

}  // namespace

extern "C" {

int mhla_forward(const void* q, const void* k, const void* v, const float* W, float* out, int64_t B, int64_t H,
                 int64_t N, int64_t d, int64_t M, int causal, mhla_stream_t stream) {
    return forward_impl(mhla::kDtypeBF16, q, k, v, W, out, B, H, N, d, M, causal ? MHLA_OPT_CAUSAL : 0u, nullptr,
                        nullptr, 0, stream);
}

int mhla_forward_noalloc(const void* q, const void* k, const void* v, const float* W, float* out, int64_t B,
                         int64_t H, int64_t N, int64_t d, int64_t M, int causal, mhla_stream_t stream) {
    return forward_impl(mhla::kDtypeBF16, q, k, v, W, out, B, H, N, d, M, causal ? MHLA_OPT_CAUSAL : 0u, nullptr,
                        nullptr, 0, stream, true, kNoAllocScratchBytes);
}

int mhla_forward_f32(const float* q, const float* k, const float* v, const float* W, float* out, int64_t B,
                     int64_t H, int64_t N, int64_t d, int64_t M, int causal, mhla_stream_t stream) {
    return forward_impl(mhla::kDtypeF32, q, k, v, W, out, B, H, N, d, M, causal ? MHLA_OPT_CAUSAL : 0u, nullptr,
                        nullptr, 0, stream);
}

int mhla_forward_ex(const void* q, const void* k, const void* v, int dtype, const float* W, void* out, int64_t B,
                    int64_t H, int64_t N, int64_t d, int64_t M, unsigned options, mhla_stream_t stream) {
    if (dtype != MHLA_DTYPE_BF16 && dtype != MHLA_DTYPE_F32) return fail(MHLA_ERR_INVALID_ARG, "bad dtype %d", dtype);
    return forward_impl(dtype, q, k, v, W, out, B, H, N, d, M, options, nullptr, nullptr, 0, stream);
}

int mhla_forward_blocks(const void* q, const void* k, const void* v, int dtype, const float* W, void* out,
                        int64_t B, int64_t H, int64_t N, int64_t d, int64_t M, const int32_t* order,
                        const int32_t* offsets, int64_t max_block, unsigned options, mhla_stream_t stream) {
    if (dtype != MHLA_DTYPE_BF16 && dtype != MHLA_DTYPE_F32) return fail(MHLA_ERR_INVALID_ARG, "bad dtype %d", dtype);
    if (!order || !offsets) return fail(MHLA_ERR_INVALID_ARG, "order and offsets are required");
    return forward_impl(dtype, q, k, v, W, out, B, H, N, d, M, options, order, offsets, max_block, stream);
}

int64_t mhla_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int64_t M, int causal) {
    (void)causal;
    if (check_sizes(B, H, N, d, M) != MHLA_OK) return -1;
    return (int64_t)workspace_bytes(mhla::kDtypeBF16, B * H, N / M, d, M);
}

int mhla_forward_path(int64_t B, int64_t H, int64_t N, int64_t d, int64_t M, int causal, int dtype) {
    if (check_sizes(B, H, N, d, M) != MHLA_OK) return -1;
    if (dtype != MHLA_DTYPE_BF16 && dtype != MHLA_DTYPE_F32) return fail(MHLA_ERR_INVALID_ARG, "bad dtype %d", dtype);
    return forward_path(B, H, N, d, M, causal, dtype);
}

int64_t mhla_summary_floats(int64_t d) { return d >= 1 ? summary_floats(d) : -1; }

int mhla_block_summaries(const void* k, const void* v, int dtype, float* S, int64_t B, int64_t H, int64_t N,
                         int64_t d, int64_t M, mhla_stream_t stream) {
    int st = check_sizes(B, H, N, d, M);
    if (st) return st;
    if (dtype != MHLA_DTYPE_BF16 && dtype != MHLA_DTYPE_F32) return fail(MHLA_ERR_INVALID_ARG, "bad dtype %d", dtype);
    if ((st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) || (st = check_ptr(S, "S"))) return st;
    const size_t esz = dtype == MHLA_DTYPE_F32 ? 4 : 2;
    const size_t in_bytes = (size_t)(B * H * N * d) * esz;
    const size_t s_bytes = (size_t)(M * B * H * summary_floats(d)) * 4;
    if (overlaps(S, s_bytes, k, in_bytes) || overlaps(S, s_bytes, v, in_bytes))
        return fail(MHLA_ERR_INVALID_ARG, "S overlaps an input");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    void* partial = nullptr;
    const size_t pbytes = mhla::summary_partial_bytes(dtype, B * H, N / M, (int)d, M);
    bool owned = false;
    if (pbytes && (st = stream_workspace(pbytes, s, &partial, &owned))) return st;
    const mhla::BlockLayout equal{nullptr, nullptr};
    hipError_t e = mhla::launch_summaries(dtype, k, v, S, B * H, N, (int)d, M, 0, equal, N / M,
                                          static_cast<float*>(partial), s);
    const hipError_t fe = release_workspace(partial, owned, s);
    if (e != hipSuccess) return hip_fail(e, "summary kernel");
    if (fe != hipSuccess) return hip_fail(fe, "workspace release");
    return ok();
}

int mhla_mix_summaries(const float* S, const float* W, float* St, int64_t BH, int64_t d, int64_t M, int causal,
                       int precise, mhla_stream_t stream) {
    int st = check_sizes(BH, 1, M, d, M);
    if (st) return st;
    if ((st = check_ptr(S, "S")) || (st = check_ptr(W, "W")) || (st = check_ptr(St, "St"))) return st;
    const size_t s_bytes = (size_t)(M * BH * summary_floats(d)) * 4;
    if (overlaps(St, s_bytes, S, s_bytes) || overlaps(St, s_bytes, W, (size_t)(M * M) * 4))
        return fail(MHLA_ERR_INVALID_ARG, "St overlaps an input");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    void* frags = nullptr;
    const size_t fbytes = precise ? 0 : mhla::mix_fragment_bytes(M);
    bool owned = false;
    if (fbytes && (st = stream_workspace(fbytes, s, &frags, &owned))) return st;
    hipError_t e = mhla::launch_mix(S, W, St, BH, (int)d, M, causal != 0, precise != 0, 0, frags, s);
    const hipError_t fe = release_workspace(frags, owned, s);
    if (e != hipSuccess) return hip_fail(e, "mixing kernel");
    if (fe != hipSuccess) return hip_fail(fe, "workspace release");
    return ok();
}

int mhla_output(const void* q, const void* k, const void* v, int dtype, const float* St, const float* W, float* out,
                int64_t B, int64_t H, int64_t N, int64_t d, int64_t M, int causal, mhla_stream_t stream) {
    int st = check_sizes(B, H, N, d, M);
    if (st) return st;
    if (dtype != MHLA_DTYPE_BF16 && dtype != MHLA_DTYPE_F32) return fail(MHLA_ERR_INVALID_ARG, "bad dtype %d", dtype);
    if ((st = check_ptr(q, "q")) || (st = check_ptr(St, "St")) || (st = check_ptr(out, "out"))) return st;
    if (causal && ((st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) || (st = check_ptr(W, "W")))) return st;
    const size_t esz = dtype == MHLA_DTYPE_F32 ? 4 : 2;
    const size_t in_bytes = (size_t)(B * H * N * d) * esz;
    const size_t out_bytes = (size_t)(B * H * N * d) * 4;
    const size_t s_bytes = (size_t)(M * B * H * summary_floats(d)) * 4;
    if (overlaps(out, out_bytes, q, in_bytes) || overlaps(out, out_bytes, St, s_bytes) ||
        (causal && (overlaps(out, out_bytes, k, in_bytes) || overlaps(out, out_bytes, v, in_bytes) ||
                    overlaps(out, out_bytes, W, (size_t)(M * M) * 4))))
        return fail(MHLA_ERR_INVALID_ARG, "out overlaps an input");
    const mhla::OutSpec os{out, 0, 1};
    const mhla::BlockLayout equal{nullptr, nullptr};
    hipError_t e = mhla::launch_output(dtype, q, k, v, St, W, os, B * H, N, (int)d, M, causal != 0, 0, equal, N / M,
                                       reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "output kernel");
    return ok();
}

int64_t mhla_backward_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int64_t M, int causal) {
    if (check_sizes(B, H, N, d, M) != MHLA_OK) return -1;
    const size_t f = mhla::backward_workspace_floats(B * H, N, (int)d, M, causal != 0) * sizeof(float);
    return (int64_t)((f + 15) / 16 * 16 + mhla::mix_fragment_bytes(M));
}

int mhla_backward(const void* q, const void* k, const void* v, int dtype, const float* W, const float* dy,
                  float* dq, float* dk, float* dv, float* dW, int64_t B, int64_t H, int64_t N, int64_t d,
                  int64_t M, int causal, mhla_stream_t stream) {
    return mhla_backward_ex(q, k, v, dtype, W, dy, dq, dk, dv, dW, B, H, N, d, M, causal ? MHLA_OPT_CAUSAL : 0,
                            stream);
}

int mhla_backward_ex(const void* q, const void* k, const void* v, int dtype, const float* W, const float* dy,
                     float* dq, float* dk, float* dv, float* dW, int64_t B, int64_t H, int64_t N, int64_t d,
                     int64_t M, unsigned options, mhla_stream_t stream_) {
    if (options & ~kKnownOptions) return fail(MHLA_ERR_INVALID_ARG, "unknown option bits 0x%x", options & ~kKnownOptions);
    if (options & (MHLA_OPT_OUT_BF16 | MHLA_OPT_W_PER_HEAD))
        return fail(MHLA_ERR_UNSUPPORTED, "the backward pass takes MHLA_OPT_CAUSAL and MHLA_OPT_NO_NORMALIZER only");
    const int causal = (options & MHLA_OPT_CAUSAL) != 0;
    const bool normalize = (options & MHLA_OPT_NO_NORMALIZER) == 0;
    int st = check_sizes(B, H, N, d, M);
    if (st) return st;
    if (dtype != MHLA_DTYPE_BF16 && dtype != MHLA_DTYPE_F32) return fail(MHLA_ERR_INVALID_ARG, "bad dtype %d", dtype);
    if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
        (st = check_ptr(W, "W")) || (st = check_ptr(dy, "dy")) || (st = check_ptr(dq, "dq")) ||
        (st = check_ptr(dk, "dk")) || (st = check_ptr(dv, "dv")) || (st = check_ptr(dW, "dW")))
        return st;
    const size_t esz = dtype == MHLA_DTYPE_F32 ? 4 : 2;
    const size_t in_bytes = (size_t)(B * H * N * d) * esz;
    const size_t g_bytes = (size_t)(B * H * N * d) * 4;
    const size_t w_bytes = (size_t)(M * M) * 4;
    const void* ins[5] = {q, k, v, W, dy};
    const size_t in_sz[5] = {in_bytes, in_bytes, in_bytes, w_bytes, g_bytes};
    const void* outs[4] = {dq, dk, dv, dW};
    const size_t out_sz[4] = {g_bytes, g_bytes, g_bytes, w_bytes};
    for (int o = 0; o < 4; ++o) {
        for (int i = 0; i < 5; ++i)
            if (overlaps(outs[o], out_sz[o], ins[i], in_sz[i]))
                return fail(MHLA_ERR_INVALID_ARG, "a gradient output overlaps an input");
        for (int o2 = 0; o2 < o; ++o2)
            if (overlaps(outs[o], out_sz[o], outs[o2], out_sz[o2]))
                return fail(MHLA_ERR_INVALID_ARG, "gradient outputs overlap each other");
    }
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    const size_t fbytes = (mhla::backward_workspace_floats(B * H, N, (int)d, M, causal != 0) * sizeof(float) + 15) /
                          16 * 16;
    const size_t total = fbytes + mhla::mix_fragment_bytes(M);
    void* ws = nullptr;
    bool owned = false;
    if ((st = stream_workspace(total, stream, &ws, &owned))) return st;
    hipError_t e = mhla::launch_backward(dtype, q, k, v, W, dy, dq, dk, dv, dW, B * H, N, (int)d, M, causal != 0, normalize,
                                         static_cast<float*>(ws), static_cast<char*>(ws) + fbytes, stream);
    const hipError_t fe = release_workspace(ws, owned, stream);
    if (e != hipSuccess) return hip_fail(e, "backward kernels");
    if (fe != hipSuccess) return hip_fail(fe, "workspace release");
    return ok();
}

int64_t mhla_decode_state_bytes(int64_t B, int64_t H, int64_t d, int64_t M) {
    if (check_sizes(B, H, M, d, M) != MHLA_OK) return -1;
    return ((M + 1) * summary_floats(d) + d) * B * H * 4;
}

int mhla_decode_step(const void* q, const void* k, const void* v, int dtype, const float* W, float* state,
                     float* out, int64_t B, int64_t H, int64_t d, int64_t M, int64_t C, int64_t t,
                     mhla_stream_t stream) {
    return mhla_decode_step_ex(q, k, v, dtype, W, state, out, B, H, d, M, C, t, MHLA_OPT_CAUSAL, stream);
}

int mhla_decode_step_ex(const void* q, const void* k, const void* v, int dtype, const float* W, float* state,
                        float* out, int64_t B, int64_t H, int64_t d, int64_t M, int64_t C, int64_t t,
                        unsigned options, mhla_stream_t stream) {
    if (options & ~kKnownOptions) return fail(MHLA_ERR_INVALID_ARG, "unknown option bits 0x%x", options & ~kKnownOptions);
    if (options & MHLA_OPT_OUT_BF16) return fail(MHLA_ERR_UNSUPPORTED, "decoding writes float32 only");
    const bool normalize = (options & MHLA_OPT_NO_NORMALIZER) == 0;
    const int heads = (options & MHLA_OPT_W_PER_HEAD) ? (int)H : 0;
    if (C < 1) return fail(MHLA_ERR_INVALID_ARG, "C=%lld must be >= 1", (long long)C);
    if (M > (((int64_t)1 << 30) / C)) return fail(MHLA_ERR_UNSUPPORTED, "M*C too large");
    int st = check_sizes(B, H, M * C, d, M);
    if (st) return st;
    if (dtype != MHLA_DTYPE_BF16 && dtype != MHLA_DTYPE_F32) return fail(MHLA_ERR_INVALID_ARG, "bad dtype %d", dtype);
    if (t < 0 || t / C >= M)
        return fail(MHLA_ERR_INVALID_ARG, "token t=%lld is outside the M*C=%lld tokens", (long long)t,
                    (long long)(M * C));
    if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
        (st = check_ptr(W, "W")) || (st = check_ptr(state, "state")) || (st = check_ptr(out, "out")))
        return st;
    const size_t esz = dtype == MHLA_DTYPE_F32 ? 4 : 2;
    const size_t in_bytes = (size_t)(B * H * d) * esz;
    const size_t out_bytes = (size_t)(B * H * d) * 4;
    const size_t st_bytes = (size_t)mhla_decode_state_bytes(B, H, d, M);
    const size_t w_bytes = (size_t)(M * M) * 4 * (heads > 0 ? (size_t)H : 1);
    if (overlaps(out, out_bytes, q, in_bytes) || overlaps(out, out_bytes, k, in_bytes) ||
        overlaps(out, out_bytes, v, in_bytes) || overlaps(out, out_bytes, W, w_bytes) ||
        overlaps(out, out_bytes, state, st_bytes))
        return fail(MHLA_ERR_INVALID_ARG, "out overlaps an input or the state");
    if (overlaps(state, st_bytes, q, in_bytes) || overlaps(state, st_bytes, k, in_bytes) ||
        overlaps(state, st_bytes, v, in_bytes) || overlaps(state, st_bytes, W, w_bytes))
        return fail(MHLA_ERR_INVALID_ARG, "state overlaps an input");
    hipError_t e = mhla::launch_decode_step(dtype, q, k, v, W, state, out, B * H, (int)d, M, C, t, normalize, heads,
                                            reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "decode kernels");
    return ok();
}

int mhla_unpack_summaries(const float* packed, int64_t count, int64_t d, float* S, float* z) {
    if (!packed || !S || !z || count < 0) return fail(MHLA_ERR_INVALID_ARG, "bad unpack arguments");
    if (d != 16 && d != 32 && d != 64) return fail(MHLA_ERR_UNSUPPORTED, "d=%lld is not one of 16, 32, 64", (long long)d);
    const int P = (int)(d / 16);
    const int64_t L = summary_floats(d);
    for (int64_t u = 0; u < count; ++u) {
        const float* src = packed + u * L;
        for (int r = 0; r < d; ++r) {
            for (int c = 0; c < d; ++c) S[(u * d + r) * d + c] = src[mhla::packed_index(P, r, c)];
            z[u * d + r] = src[d * d + r];
        }
    }
    return ok();
}

int mhla_release_workspace(mhla_stream_t stream) {
    return drop_stream_workspace(reinterpret_cast<hipStream_t>(stream));
}

void mhla_debug_fail_workspace(int count) { g_fail_workspace.store(count > 0 ? count : 0); }

const char* mhla_status_string(int status) {
    switch (status) {
        case MHLA_OK: return "MHLA_OK";
        case MHLA_ERR_INVALID_ARG: return "MHLA_ERR_INVALID_ARG";
        case MHLA_ERR_UNSUPPORTED: return "MHLA_ERR_UNSUPPORTED";
        case MHLA_ERR_NO_MEMORY: return "MHLA_ERR_NO_MEMORY";
        case MHLA_ERR_HIP: return "MHLA_ERR_HIP";
        default: return "MHLA_ERR_UNKNOWN";
    }
}

const char* mhla_last_error(void) { return g_err; }

const char* mhla_version(void) { return "mhla-gfx950 0.1.0"; }

}  // extern "C"
