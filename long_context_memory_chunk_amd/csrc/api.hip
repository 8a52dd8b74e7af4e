// Host side of the C ABI: context, argument validation, dispatch, and the
// host-store gather.  Every entry point validates its arguments before it
// enqueues anything and reports errors through msa_status plus a
// thread-local message; no exception leaves this file.
#include <dlfcn.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "common.hpp"
#include "launch.hpp"

namespace msa {
bool route_generic_supported(int Hkv);
bool attn_supported_group(int Hq, int Hkv);
}  // namespace msa

namespace {

thread_local std::string g_err;

// Library-held scratch for msa_sparse_attn_noalloc: one array per device
// (each device holds its own copy, at its own address, for the life of the
// process).  Host code never uses the array's name as an address: the device
// address is looked up once per device, with that device current, and kept
// in g_scratch_addr (and in every context on that device).
static __device__ __align__(256) unsigned char scratch[MSA_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_addr;

// msa_gather submits its copies with hipMemcpyBatchAsync when the HIP runtime
// loaded in the process provides it (looked up at run time: an older runtime
// in the same process, e.g. one bundled with a framework, may lack it) and
// MSA_GATHER_BATCH=0 is not set; otherwise one hipMemcpyAsync per copy.
const bool g_gather_batch = [] {
    const char* v = std::getenv("MSA_GATHER_BATCH");
    return !(v && v[0] == '0');
}();

using BatchCopyFn = hipError_t (*)(void**, void**, size_t*, size_t, hipMemcpyAttributes*, size_t*,
                                   size_t, size_t*, hipStream_t);

BatchCopyFn batch_copy_fn() {
    static const BatchCopyFn fn =
        reinterpret_cast<BatchCopyFn>(dlsym(RTLD_DEFAULT, "hipMemcpyBatchAsync"));
    return fn;
}

msa_status fail(msa_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

msa_status ok() {
    g_err.clear();
    return MSA_OK;
}

msa_status hip_fail(hipError_t e, const char* what) {
    return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

size_t dtype_bytes(msa_dtype dt) { return dt == MSA_BF16 ? 2 : 4; }
bool dtype_ok(msa_dtype dt) { return dt == MSA_F32 || dt == MSA_BF16; }

// Makes the context's device current for the duration of a call.  It also
// clears a stale, non-sticky error left by an unrelated earlier HIP call (a
// failed allocation, say), so the launch checks of this call report only
// errors of this call.
struct DeviceGuard {
    int prev = -1;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev) {
        (void)hipGetLastError();
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != dev) err = hipSetDevice(dev);
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

// Document-local positions run from 0 to max_doc_len - 1, and every one of
// them must have a row in the context's RoPE table.
msa_status check_doc_len(const char* fn, const msa_ctx* ctx, int64_t n_docs, int64_t T, int64_t max_doc_len) {
    if (n_docs == 0) return MSA_OK;
    if (max_doc_len < 1 || max_doc_len > T)
        return fail(MSA_ERR_INVALID_ARG, "%s: max_doc_len %lld outside [1, T = %lld]", fn, (long long)max_doc_len,
                    (long long)T);
    if (max_doc_len > ctx->max_pos)
        return fail(MSA_ERR_INVALID_ARG,
                    "%s: a document of %lld tokens needs RoPE positions up to %lld, but the context's "
                    "max_pos is %d", fn, (long long)max_doc_len, (long long)(max_doc_len - 1), ctx->max_pos);
    return MSA_OK;
}

// Checks of the device gather's arguments (msa_gather_device, msa_gather_attn).
msa_status check_gather_device(const char* fn, const msa_ctx* ctx, const void* host_KVbar, size_t row_bytes,
                               int64_t n_rows_host, const int64_t* doc_chunk_off, int64_t n_docs,
                               const int32_t* ids, int64_t B, int top_k, const void* dst_KVmem, int64_t cap_rows,
                               const int64_t* mem_off) {
    if (!ctx) return fail(MSA_ERR_INVALID_ARG, "%s: ctx is NULL", fn);
    if (!host_KVbar || !doc_chunk_off || !ids || !dst_KVmem || !mem_off)
        return fail(MSA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (row_bytes == 0 || row_bytes % 16 || n_rows_host < 0 || n_docs < 1 || cap_rows < 0)
        return fail(MSA_ERR_INVALID_ARG, "%s: bad size (row_bytes must be a multiple of 16)", fn);
    if (B < 1 || B > msa::kMaxGatherB)
        return fail(MSA_ERR_UNSUPPORTED, "%s: B must be in [1, %d]", fn, msa::kMaxGatherB);
    if (top_k < 1 || top_k > MSA_MAX_TOPK || top_k > n_docs)
        return fail(MSA_ERR_INVALID_ARG, "%s: top_k %d outside [1, min(n_docs, %d)]", fn, top_k, MSA_MAX_TOPK);
    if (!aligned16(host_KVbar) || !aligned16(dst_KVmem))
        return fail(MSA_ERR_INVALID_ARG, "%s: host store and destination must be 16-byte aligned", fn);
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof(attr));
    const hipError_t e = hipPointerGetAttributes(&attr, host_KVbar);
    if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
        (void)hipGetLastError();
        return fail(MSA_ERR_INVALID_ARG, "%s: host store is not pinned host memory (use hipHostMalloc)", fn);
    }
    return MSA_OK;
}

}  // namespace

extern "C" {

int msa_abi_version(void) { return MSA_ABI_VERSION; }

const char* msa_last_error(void) { return g_err.c_str(); }

const char* msa_status_string(msa_status s) {
    switch (s) {
        case MSA_OK: return "MSA_OK";
        case MSA_ERR_INVALID_ARG: return "MSA_ERR_INVALID_ARG";
        case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED";
        case MSA_ERR_HIP: return "MSA_ERR_HIP";
        case MSA_ERR_WORKSPACE: return "MSA_ERR_WORKSPACE";
    }
    return "MSA_STATUS_UNKNOWN";
}

msa_status msa_ctx_create(int device, int head_dim, double rope_theta, int max_pos, msa_ctx** out) {
    if (!out) return fail(MSA_ERR_INVALID_ARG, "msa_ctx_create: out is NULL");
    if (head_dim != 64 && head_dim != 128)
        return fail(MSA_ERR_UNSUPPORTED, "msa_ctx_create: head_dim %d (supported: 64, 128)", head_dim);
    if (!(rope_theta > 1.0) || !std::isfinite(rope_theta))
        return fail(MSA_ERR_INVALID_ARG, "msa_ctx_create: rope_theta must be finite and > 1");
    if (max_pos < 1 || max_pos > (1 << 22))
        return fail(MSA_ERR_INVALID_ARG, "msa_ctx_create: max_pos %d outside [1, 2^22]", max_pos);
    int n_dev = 0;
    hipError_t e = hipGetDeviceCount(&n_dev);
    if (e != hipSuccess) return hip_fail(e, "msa_ctx_create: hipGetDeviceCount");
    if (device < 0 || device >= n_dev)
        return fail(MSA_ERR_INVALID_ARG, "msa_ctx_create: device %d (have %d)", device, n_dev);
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess) return hip_fail(e, "msa_ctx_create: hipGetDeviceProperties");
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(MSA_ERR_UNSUPPORTED, "msa_ctx_create: device %d is %s, built for gfx950", device,
                    prop.gcnArchName);

    // cos/sin table from float64 angles pos * theta^(-2i/d), stored as float32
    const int half = head_dim / 2;
    std::vector<float2> table;
    try {
        table.resize(size_t(max_pos) * half);
    } catch (const std::bad_alloc&) {
        return fail(MSA_ERR_INVALID_ARG, "msa_ctx_create: host allocation of the RoPE table failed");
    }
    std::vector<double> inv(half);
    for (int i = 0; i < half; ++i) inv[i] = std::pow(rope_theta, -2.0 * double(i) / double(head_dim));
    for (int p = 0; p < max_pos; ++p)
        for (int i = 0; i < half; ++i) {
            const double a = double(p) * inv[i];
            table[size_t(p) * half + i] = make_float2(float(std::cos(a)), float(std::sin(a)));
        }

    DeviceGuard dg(device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "msa_ctx_create: hipSetDevice");
    float2* d_table = nullptr;
    e = hipMalloc(&d_table, table.size() * sizeof(float2));
    if (e != hipSuccess) return hip_fail(e, "msa_ctx_create: hipMalloc of the RoPE table");
    e = hipMemcpy(d_table, table.data(), table.size() * sizeof(float2), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(d_table);
        return hip_fail(e, "msa_ctx_create: hipMemcpy of the RoPE table");
    }
    msa_ctx* c = new (std::nothrow) msa_ctx;
    if (!c) {
        (void)hipFree(d_table);
        return fail(MSA_ERR_INVALID_ARG, "msa_ctx_create: out of host memory");
    }
    c->device = device;
    c->head_dim = head_dim;
    c->theta = rope_theta;
    c->max_pos = max_pos;
    c->num_cus = prop.multiProcessorCount;
    c->rope_cs = d_table;
    c->prof_start = nullptr;
    c->prof_stop = nullptr;
    c->scratch = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        auto it = g_scratch_addr.find(device);
        if (it == g_scratch_addr.end()) {
            void* addr = nullptr;
            e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));   // the device is current (DeviceGuard)
            if (e != hipSuccess || !addr) {
                delete c;
                (void)hipFree(d_table);
                return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                                "msa_ctx_create: hipGetSymbolAddress of the scratch array");
            }
            it = g_scratch_addr.emplace(device, addr).first;
        }
        c->scratch = it->second;
    }
    *out = c;
    return ok();
}

msa_status msa_ctx_destroy(msa_ctx* ctx) {
    if (!ctx) return ok();
    DeviceGuard dg(ctx->device);
    hipError_t e = hipDeviceSynchronize();
    hipError_t e2 = hipFree(ctx->rope_cs);
    delete ctx;
    if (e != hipSuccess) return hip_fail(e, "msa_ctx_destroy: hipDeviceSynchronize");
    if (e2 != hipSuccess) return hip_fail(e2, "msa_ctx_destroy: hipFree");
    return ok();
}

msa_status msa_chunk_offsets(const int64_t* doc_tok_off, int64_t n_docs, int chunk_len,
                             int64_t* doc_chunk_off, int64_t* max_doc_len) {
    if (!doc_tok_off || !doc_chunk_off) return fail(MSA_ERR_INVALID_ARG, "msa_chunk_offsets: NULL pointer");
    if (n_docs < 0) return fail(MSA_ERR_INVALID_ARG, "msa_chunk_offsets: n_docs < 0");
    if (chunk_len < 1) return fail(MSA_ERR_INVALID_ARG, "msa_chunk_offsets: chunk_len < 1");
    if (doc_tok_off[0] != 0) return fail(MSA_ERR_INVALID_ARG, "msa_chunk_offsets: doc_tok_off[0] != 0");
    for (int64_t d = 0; d < n_docs; ++d)
        if (doc_tok_off[d + 1] <= doc_tok_off[d])
            return fail(MSA_ERR_INVALID_ARG, "msa_chunk_offsets: document %lld has no token",
                        (long long)d);
    doc_chunk_off[0] = 0;
    int64_t longest = 0;
    for (int64_t d = 0; d < n_docs; ++d) {
        const int64_t len = doc_tok_off[d + 1] - doc_tok_off[d];
        doc_chunk_off[d + 1] = doc_chunk_off[d] + (len + chunk_len - 1) / chunk_len;
        longest = std::max(longest, len);
    }
    if (max_doc_len) *max_doc_len = longest;
    return ok();
}

msa_status msa_encode_pool(msa_ctx* ctx, msa_dtype dt, const void* K, const void* V, const void* Kr,
                           const int64_t* doc_tok_off, const int64_t* doc_chunk_off, int64_t n_docs,
                           int64_t T, int64_t N, int Hkv, int chunk_len, int64_t max_doc_len, void* KVbar,
                           void* Krbar, hipStream_t stream) {
    const char* fn = "msa_encode_pool";
    if (!ctx) return fail(MSA_ERR_INVALID_ARG, "%s: ctx is NULL", fn);
    if (!dtype_ok(dt)) return fail(MSA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, int(dt));
    if (n_docs < 0 || T < 0 || N < 0) return fail(MSA_ERR_INVALID_ARG, "%s: negative size", fn);
    if (Hkv < 1) return fail(MSA_ERR_INVALID_ARG, "%s: Hkv < 1", fn);
    if (chunk_len < 1) return fail(MSA_ERR_INVALID_ARG, "%s: chunk_len < 1", fn);
    if (n_docs > 0x7FFFFFFF) return fail(MSA_ERR_UNSUPPORTED, "%s: n_docs > 2^31-1", fn);
    if (n_docs > T) return fail(MSA_ERR_INVALID_ARG, "%s: %lld documents but %lld tokens", fn,
                                (long long)n_docs, (long long)T);
    if (n_docs > N) return fail(MSA_ERR_INVALID_ARG, "%s: %lld documents but %lld chunk rows", fn,
                                (long long)n_docs, (long long)N);
    if (N > T) return fail(MSA_ERR_INVALID_ARG, "%s: more chunk rows than tokens", fn);
    if (msa_status s = check_doc_len(fn, ctx, n_docs, T, max_doc_len)) return s;
    if (n_docs > 0 && (!K || !V || !Kr || !doc_tok_off || !doc_chunk_off || !KVbar || !Krbar))
        return fail(MSA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (n_docs > 0 && (!aligned16(K) || !aligned16(V) || !aligned16(Kr) || !aligned16(KVbar) ||
                       !aligned16(Krbar)))
        return fail(MSA_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
    DeviceGuard dg(ctx->device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "msa_encode_pool: hipSetDevice");
    hipError_t e = msa::launch_encode(ctx, dt, K, V, Kr, doc_tok_off, doc_chunk_off, n_docs, T, N, Hkv,
                                      chunk_len, max_doc_len, KVbar, Krbar, stream);
    if (e != hipSuccess) return hip_fail(e, "msa_encode_pool: launch");
    return ok();
}

msa_status msa_encode_pool_bwd(msa_ctx* ctx, msa_dtype dt, const void* dKVbar, const void* dKrbar,
                               const int64_t* doc_tok_off, const int64_t* doc_chunk_off, int64_t n_docs, int64_t T,
                               int64_t N, int Hkv, int chunk_len, int64_t max_doc_len, void* dK, void* dV,
                               void* dKr, hipStream_t stream) {
    const char* fn = "msa_encode_pool_bwd";
    if (!ctx) return fail(MSA_ERR_INVALID_ARG, "%s: ctx is NULL", fn);
    if (!dtype_ok(dt)) return fail(MSA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, int(dt));
    if (n_docs < 0 || T < 0 || N < 0) return fail(MSA_ERR_INVALID_ARG, "%s: negative size", fn);
    if (Hkv < 1) return fail(MSA_ERR_INVALID_ARG, "%s: Hkv < 1", fn);
    if (chunk_len < 1) return fail(MSA_ERR_INVALID_ARG, "%s: chunk_len < 1", fn);
    if (n_docs > 0x7FFFFFFF) return fail(MSA_ERR_UNSUPPORTED, "%s: n_docs > 2^31-1", fn);
    if (n_docs > T || n_docs > N || N > T)
        return fail(MSA_ERR_INVALID_ARG, "%s: need n_docs <= N <= T (%lld, %lld, %lld)", fn, (long long)n_docs,
                    (long long)N, (long long)T);
    if (msa_status s = check_doc_len(fn, ctx, n_docs, T, max_doc_len)) return s;
    if (n_docs > 0 && (!dKVbar || !dKrbar || !doc_tok_off || !doc_chunk_off || !dK || !dV || !dKr))
        return fail(MSA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (n_docs > 0 && (!aligned16(dKVbar) || !aligned16(dKrbar) || !aligned16(dK) || !aligned16(dV) ||
                       !aligned16(dKr)))
        return fail(MSA_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
    DeviceGuard dg(ctx->device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "msa_encode_pool_bwd: hipSetDevice");
    hipError_t e = msa::launch_encode_bwd(ctx, dt, dKVbar, dKrbar, doc_tok_off, doc_chunk_off, n_docs, T, N, Hkv,
                                          chunk_len, max_doc_len, dK, dV, dKr, stream);
    if (e != hipSuccess) return hip_fail(e, "msa_encode_pool_bwd: launch");
    return ok();
}

size_t msa_route_workspace_size(msa_dtype dt, int64_t B, int Tq, int Hq, int Hkv, int64_t N,
                                int64_t n_docs, int top_k) {
    if (B < 1 || Tq < 1 || Hkv < 1 || N < 0 || n_docs < 1 || top_k < 1) return 0;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess) cus = prop.multiProcessorCount;
    }
    // sized for head_dim 128 so one workspace serves both head dims
    return msa::route_workspace(dt, B, Tq, Hq, Hkv, 128, N, n_docs, top_k, cus);
}

msa_status msa_route(msa_ctx* ctx, msa_dtype dt, const void* Qr, int64_t B, int Tq, int Hq,
                     const void* Krbar, int64_t N, int Hkv, const int64_t* doc_chunk_off,
                     int64_t n_docs, int top_k, int32_t* out_ids, float* out_scores, float* out_chunk,
                     float* out_doc, void* workspace, size_t ws_bytes, hipStream_t stream) {
    const char* fn = "msa_route";
    if (!ctx) return fail(MSA_ERR_INVALID_ARG, "%s: ctx is NULL", fn);
    if (!dtype_ok(dt)) return fail(MSA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, int(dt));
    if (B < 1 || Tq < 1 || Hq < 1 || Hkv < 1)
        return fail(MSA_ERR_INVALID_ARG, "%s: B, Tq, Hq and Hkv must be >= 1", fn);
    if (Hq % Hkv) return fail(MSA_ERR_INVALID_ARG, "%s: Hq %% Hkv != 0 (%d, %d)", fn, Hq, Hkv);
    if (n_docs < 1) return fail(MSA_ERR_INVALID_ARG, "%s: n_docs < 1", fn);
    if (n_docs > 0xFFFFFFF0LL) return fail(MSA_ERR_UNSUPPORTED, "%s: n_docs >= 2^32-16", fn);
    if (N < n_docs) return fail(MSA_ERR_INVALID_ARG, "%s: N (%lld) < n_docs (%lld)", fn, (long long)N,
                                (long long)n_docs);
    if (top_k < 1 || top_k > MSA_MAX_TOPK || top_k > n_docs)
        return fail(MSA_ERR_INVALID_ARG, "%s: top_k %d outside [1, min(n_docs, %d)]", fn, top_k,
                    MSA_MAX_TOPK);
    if (B > 65535) return fail(MSA_ERR_UNSUPPORTED, "%s: B > 65535", fn);
    if (B * Tq * Hkv > 0x7FFFFFFF) return fail(MSA_ERR_UNSUPPORTED, "%s: B*Tq*Hkv too large", fn);
    if (!Qr || !Krbar || !doc_chunk_off || !out_ids)
        return fail(MSA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned16(Krbar)) return fail(MSA_ERR_INVALID_ARG, "%s: Krbar must be 16-byte aligned", fn);
    if (!msa::route_generic_supported(Hkv)) return fail(MSA_ERR_UNSUPPORTED, "%s: Hkv > 32", fn);
    const size_t need = msa::route_workspace(dt, B, Tq, Hq, Hkv, ctx->head_dim, N, n_docs, top_k,
                                             ctx->num_cus);
    if (!workspace || !aligned256(workspace) || ws_bytes < need)
        return fail(MSA_ERR_WORKSPACE, "%s: workspace needs %zu bytes, 256-aligned (got %zu)", fn, need,
                    ws_bytes);
    msa::RouteArgs a{dt, Qr, B, Tq, Hq, Hkv, ctx->head_dim, Krbar, N, doc_chunk_off, n_docs, top_k,
                     out_ids, out_scores, out_chunk, out_doc, workspace, ws_bytes, ctx->num_cus,
                     ctx->prof_start, ctx->prof_stop};
    ctx->prof_start = ctx->prof_stop = nullptr;
    DeviceGuard dg(ctx->device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "msa_route: hipSetDevice");
    hipError_t e = msa::launch_route(a, stream);
    if (e != hipSuccess) return hip_fail(e, "msa_route: launch");
    return ok();
}

size_t msa_route_bwd_workspace_size(int64_t B, int Tq, int Hq, int Hkv, int64_t N, int64_t n_docs) {
    if (B < 1 || Tq < 1 || Hq < 1 || Hkv < 1 || N < 1 || n_docs < 1) return 0;
    return msa::route_bwd_workspace(B, Tq, Hq, Hkv, 128, N, n_docs);   // sized for head dim 128
}

msa_status msa_route_bwd(msa_ctx* ctx, msa_dtype dt, const void* Qr, int64_t B, int Tq, int Hq,
                         const void* Krbar, int64_t N, int Hkv, const int64_t* doc_chunk_off, int64_t n_docs,
                         const float* dscore, float* dQr, float* dKrbar, int32_t* out_arg, void* workspace,
                         size_t ws_bytes, hipStream_t stream) {
    const char* fn = "msa_route_bwd";
    if (!ctx) return fail(MSA_ERR_INVALID_ARG, "%s: ctx is NULL", fn);
    if (!dtype_ok(dt)) return fail(MSA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, int(dt));
    if (B < 1 || Tq < 1 || Hq < 1 || Hkv < 1 || N < 1 || n_docs < 1)
        return fail(MSA_ERR_INVALID_ARG, "%s: B, Tq, Hq, Hkv, N and n_docs must be >= 1", fn);
    if (Hq % Hkv) return fail(MSA_ERR_INVALID_ARG, "%s: Hq %% Hkv != 0 (%d, %d)", fn, Hq, Hkv);
    const int RW = Hkv * ctx->head_dim;
    if (RW % 64 || RW > 2048 || (RW / 64) & (RW / 64 - 1))
        return fail(MSA_ERR_UNSUPPORTED, "%s: Hkv * head_dim must be 64 .. 2048, a power of two", fn);
    if (B > 65535 || n_docs > 0x7FFFFFFFLL || Tq > 65535)
        return fail(MSA_ERR_UNSUPPORTED, "%s: B, Tq or n_docs too large", fn);
    if (N * int64_t(Tq) > 0xFFFFFFF0LL || N > 0x7FFFFFFFLL)
        return fail(MSA_ERR_UNSUPPORTED, "%s: N * Tq must stay below 2^32", fn);
    if (!Qr || !Krbar || !doc_chunk_off || !dscore || !dQr || !dKrbar)
        return fail(MSA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (out_arg && (reinterpret_cast<uintptr_t>(out_arg) & 7u))
        return fail(MSA_ERR_INVALID_ARG, "%s: out_arg must be 8-byte aligned", fn);
    const size_t need = msa::route_bwd_workspace(B, Tq, Hq, Hkv, ctx->head_dim, N, n_docs);
    if (!workspace || !aligned256(workspace) || ws_bytes < need)
        return fail(MSA_ERR_WORKSPACE, "%s: workspace needs %zu bytes, 256-aligned (got %zu)", fn, need,
                    ws_bytes);
    msa::RouteBwdArgs a{};
    a.r = msa::RouteArgs{dt, Qr, B, Tq, Hq, Hkv, ctx->head_dim, Krbar, N, doc_chunk_off, n_docs, 1,
                         nullptr, nullptr, nullptr, nullptr, workspace, ws_bytes, ctx->num_cus, nullptr, nullptr};
    a.dscore = dscore;
    a.dQr = dQr;
    a.dKr = dKrbar;
    a.arg_out = out_arg;
    DeviceGuard dg(ctx->device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "msa_route_bwd: hipSetDevice");
    hipError_t e = msa::launch_route_bwd(a, stream);
    if (e != hipSuccess) return hip_fail(e, "msa_route_bwd: launch");
    return ok();
}

msa_status msa_route_time_next(msa_ctx* ctx, hipEvent_t start, hipEvent_t stop) {
    if (!ctx) return fail(MSA_ERR_INVALID_ARG, "msa_route_time_next: ctx is NULL");
    if ((start == nullptr) != (stop == nullptr))
        return fail(MSA_ERR_INVALID_ARG, "msa_route_time_next: give both events or neither");
    ctx->prof_start = start;
    ctx->prof_stop = stop;
    return ok();
}

msa_status msa_gather(const void* host_KVbar, size_t row_bytes, int64_t n_rows_host,
                      const int64_t* doc_chunk_off, int64_t n_docs, const int32_t* ids_host, int64_t B,
                      int top_k, void* dst_KVmem, int64_t cap_rows, int64_t* mem_off_host,
                      int64_t* mem_off_dev, hipStream_t side, hipEvent_t done) {
    const char* fn = "msa_gather";
    if (!host_KVbar || !doc_chunk_off || !ids_host || !dst_KVmem || !mem_off_host)
        return fail(MSA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (row_bytes == 0 || n_rows_host < 0 || n_docs < 1 || B < 1 || top_k < 1 || top_k > n_docs ||
        cap_rows < 0)
        return fail(MSA_ERR_INVALID_ARG, "%s: bad size", fn);
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof(attr));
    hipError_t e = hipPointerGetAttributes(&attr, host_KVbar);
    if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
        (void)hipGetLastError();
        return fail(MSA_ERR_INVALID_ARG, "%s: host store is not pinned host memory (use hipHostMalloc)",
                    fn);
    }
    // plan every copy before enqueuing any
    struct Run { int64_t src_row, dst_row, rows; };
    std::vector<Run> runs;
    runs.reserve(size_t(B) * top_k);
    std::vector<int32_t> ids(top_k);
    int64_t cur = 0;
    mem_off_host[0] = 0;
    for (int64_t b = 0; b < B; ++b) {
        std::copy(ids_host + b * top_k, ids_host + (b + 1) * top_k, ids.begin());
        std::sort(ids.begin(), ids.end());
        for (int k = 0; k < top_k; ++k) {
            const int32_t id = ids[k];
            if (id < 0 || id >= n_docs)
                return fail(MSA_ERR_INVALID_ARG, "%s: query %lld selects doc %d outside [0, %lld)", fn,
                            (long long)b, id, (long long)n_docs);
            if (k > 0 && ids[k - 1] == id)
                return fail(MSA_ERR_INVALID_ARG, "%s: query %lld selects doc %d twice", fn, (long long)b, id);
            const int64_t a = doc_chunk_off[id], z = doc_chunk_off[id + 1];
            if (a < 0 || z < a || z > n_rows_host)
                return fail(MSA_ERR_INVALID_ARG, "%s: rows of doc %d outside the host store", fn, id);
            if (cur + (z - a) > cap_rows)
                return fail(MSA_ERR_INVALID_ARG, "%s: selected rows exceed cap_rows (%lld)", fn,
                            (long long)cap_rows);
            if (!runs.empty() && runs.back().src_row + runs.back().rows == a &&
                runs.back().dst_row + runs.back().rows == cur && k > 0)
                runs.back().rows += z - a;
            else if (z > a)
                runs.push_back(Run{a, cur, z - a});
            cur += z - a;
        }
        mem_off_host[b + 1] = cur;
    }
    // one batched submission of every host->device copy (the runs, then
    // mem_off); a runtime that rejects the batch gets the copies one by one
    const char* src = static_cast<const char*>(host_KVbar);
    char* dst = static_cast<char*>(dst_KVmem);
    std::vector<void*> dsts, srcs;
    std::vector<size_t> sizes;
    dsts.reserve(runs.size() + 1);
    srcs.reserve(runs.size() + 1);
    sizes.reserve(runs.size() + 1);
    for (const Run& r : runs) {
        dsts.push_back(dst + size_t(r.dst_row) * row_bytes);
        srcs.push_back(const_cast<char*>(src) + size_t(r.src_row) * row_bytes);
        sizes.push_back(size_t(r.rows) * row_bytes);
    }
    if (mem_off_dev) {
        dsts.push_back(mem_off_dev);
        srcs.push_back(mem_off_host);
        sizes.push_back(size_t(B + 1) * sizeof(int64_t));
    }
    bool batched = false;
    if (dsts.size() > 1 && g_gather_batch) {
        if (BatchCopyFn fn = batch_copy_fn()) {
            size_t fail_idx = 0;
            e = fn(dsts.data(), srcs.data(), sizes.data(), dsts.size(), nullptr, nullptr, 0, &fail_idx, side);
            if (e == hipSuccess) batched = true;
            else (void)hipGetLastError();
        }
    }
    if (!batched) {
        for (size_t i = 0; i < dsts.size(); ++i) {
            e = hipMemcpyAsync(dsts[i], srcs[i], sizes[i], hipMemcpyHostToDevice, side);
            if (e != hipSuccess) return hip_fail(e, "msa_gather: hipMemcpyAsync");
        }
    }
    if (done) {
        e = hipEventRecord(done, side);
        if (e != hipSuccess) return hip_fail(e, "msa_gather: hipEventRecord");
    }
    return ok();
}

size_t msa_gather_device_workspace_size(int64_t B, int top_k, int64_t cap_rows) {
    if (B < 1 || top_k < 1 || cap_rows < 0) return 0;
    return msa::gather_device_workspace(B, cap_rows);
}

msa_status msa_gather_device(msa_ctx* ctx, const void* host_KVbar, size_t row_bytes, int64_t n_rows_host,
                             const int64_t* doc_chunk_off, int64_t n_docs, const int32_t* ids, int64_t B,
                             int top_k, void* dst_KVmem, int64_t cap_rows, int64_t* mem_off,
                             void* workspace, size_t ws_bytes, hipStream_t stream) {
    const char* fn = "msa_gather_device";
    msa_status s = check_gather_device(fn, ctx, host_KVbar, row_bytes, n_rows_host, doc_chunk_off, n_docs, ids, B,
                                       top_k, dst_KVmem, cap_rows, mem_off);
    if (s != MSA_OK) return s;
    const size_t need = msa::gather_device_workspace(B, cap_rows);
    if (!workspace || !aligned256(workspace) || ws_bytes < need)
        return fail(MSA_ERR_WORKSPACE, "%s: workspace needs %zu bytes, 256-aligned (got %zu)", fn, need,
                    ws_bytes);
    DeviceGuard dg(ctx->device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "msa_gather_device: hipSetDevice");
    const hipError_t e = msa::launch_gather_device(host_KVbar, row_bytes, n_rows_host, doc_chunk_off, n_docs, ids, B, top_k,
                                  dst_KVmem, cap_rows, mem_off, workspace, stream);
    if (e != hipSuccess) return hip_fail(e, "msa_gather_device: launch");
    return ok();
}

size_t msa_sparse_attn_workspace_size(msa_dtype dt, int64_t B, int Tq, int Hq, int Hkv,
                                      int64_t max_rows_per_query, int L) {
    if (B < 1 || Tq < 1 || Hq < 1 || Hkv < 1 || max_rows_per_query < 0 || L < 1) return 0;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess) cus = prop.multiProcessorCount;
    }
    return msa::attn_workspace(dt, B, Tq, Hq, Hkv, 128, max_rows_per_query, L, cus);
}

}  // extern "C"

namespace {

// Checks shared by the forward and backward attention calls.
msa_status check_attn(const char* fn, msa_ctx* ctx, msa_dtype dt, const void* Q, int64_t B, int Tq, int Hq,
                      const void* KVmem, const int64_t* mem_off, int64_t mem_rows_cap, int64_t max_rows_per_query,
                      const void* K_local, const void* V_local, int L, int Hkv, int q_offset, float scale) {
    if (!ctx) return fail(MSA_ERR_INVALID_ARG, "%s: ctx is NULL", fn);
    if (!dtype_ok(dt)) return fail(MSA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, int(dt));
    if (B < 1 || Tq < 1 || Hq < 1 || Hkv < 1 || L < 1)
        return fail(MSA_ERR_INVALID_ARG, "%s: B, Tq, Hq, Hkv and L must be >= 1", fn);
    if (Tq > L) return fail(MSA_ERR_INVALID_ARG, "%s: Tq (%d) > L (%d)", fn, Tq, L);
    if (Hq % Hkv) return fail(MSA_ERR_INVALID_ARG, "%s: Hq %% Hkv != 0 (%d, %d)", fn, Hq, Hkv);
    if (!msa::attn_supported_group(Hq, Hkv))
        return fail(MSA_ERR_UNSUPPORTED, "%s: Hq/Hkv = %d (supported 1, 2, 4, 8, 16)", fn, Hq / Hkv);
    if (q_offset < 0 || int64_t(q_offset) + L - 1 >= ctx->max_pos)
        return fail(MSA_ERR_INVALID_ARG, "%s: positions up to q_offset + L - 1 = %lld exceed max_pos %d",
                    fn, (long long)(int64_t(q_offset) + L - 1), ctx->max_pos);
    if (mem_rows_cap < 0 || max_rows_per_query < 0)
        return fail(MSA_ERR_INVALID_ARG, "%s: negative row count", fn);
    if (B * Tq > 65535LL * 1024) return fail(MSA_ERR_UNSUPPORTED, "%s: B*Tq too large", fn);
    if (!std::isfinite(scale)) return fail(MSA_ERR_INVALID_ARG, "%s: scale must be finite", fn);
    if (!Q || !mem_off || !K_local || !V_local || (mem_rows_cap > 0 && !KVmem))
        return fail(MSA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned16(K_local) || !aligned16(V_local) || (KVmem && !aligned16(KVmem)) || !aligned16(Q))
        return fail(MSA_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
    return MSA_OK;
}

msa_status sparse_attn_fwd(const char* fn, msa_ctx* ctx, msa_dtype dt, const void* Q, int64_t B, int Tq, int Hq,
                           const void* KVmem, const int64_t* mem_off, int64_t mem_rows_cap,
                           int64_t max_rows_per_query, const void* K_local, const void* V_local, int L, int Hkv,
                           int q_offset, float scale, void* O, float* lse, void* workspace, size_t ws_bytes,
                           hipStream_t stream) {
    msa_status s = check_attn(fn, ctx, dt, Q, B, Tq, Hq, KVmem, mem_off, mem_rows_cap, max_rows_per_query,
                              K_local, V_local, L, Hkv, q_offset, scale);
    if (s != MSA_OK) return s;
    if (!O) return fail(MSA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned16(O)) return fail(MSA_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
    const size_t need = msa::attn_workspace(dt, B, Tq, Hq, Hkv, ctx->head_dim, max_rows_per_query, L,
                                            ctx->num_cus);
    if (!workspace || !aligned256(workspace) || ws_bytes < need)
        return fail(MSA_ERR_WORKSPACE, "%s: workspace needs %zu bytes, 256-aligned (got %zu)", fn, need,
                    ws_bytes);
    msa::AttnArgs a{dt, Q, B, Tq, Hq, Hkv, ctx->head_dim, L, KVmem, mem_off, mem_rows_cap,
                    max_rows_per_query, K_local, V_local, q_offset, scale, O, workspace, ws_bytes,
                    ctx->rope_cs, ctx->max_pos, ctx->num_cus, lse};
    DeviceGuard dg(ctx->device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "msa_sparse_attn: hipSetDevice");
    hipError_t e = msa::launch_attn(a, stream);
    if (e != hipSuccess) return hip_fail(e, "msa_sparse_attn: launch");
    return ok();
}

}  // namespace

extern "C" {

msa_status msa_sparse_attn(msa_ctx* ctx, msa_dtype dt, const void* Q, int64_t B, int Tq, int Hq,
                           const void* KVmem, const int64_t* mem_off, int64_t mem_rows_cap,
                           int64_t max_rows_per_query, const void* K_local, const void* V_local, int L,
                           int Hkv, int q_offset, float scale, void* O, void* workspace, size_t ws_bytes,
                           hipStream_t stream) {
    return sparse_attn_fwd("msa_sparse_attn", ctx, dt, Q, B, Tq, Hq, KVmem, mem_off, mem_rows_cap,
                           max_rows_per_query, K_local, V_local, L, Hkv, q_offset, scale, O, nullptr, workspace,
                           ws_bytes, stream);
}

msa_status msa_sparse_attn_noalloc(msa_ctx* ctx, msa_dtype dt, const void* Q, int64_t B, int Tq, int Hq,
                                   const void* KVmem, const int64_t* mem_off, int64_t mem_rows_cap,
                                   int64_t max_rows_per_query, const void* K_local, const void* V_local, int L,
                                   int Hkv, int q_offset, float scale, void* O, hipStream_t stream) {
    const char* fn = "msa_sparse_attn_noalloc";
    if (!ctx) return fail(MSA_ERR_INVALID_ARG, "%s: ctx is NULL", fn);
    if (!ctx->scratch) return fail(MSA_ERR_INVALID_ARG, "%s: context has no scratch address", fn);
    msa_status s = check_attn(fn, ctx, dt, Q, B, Tq, Hq, KVmem, mem_off, mem_rows_cap, max_rows_per_query,
                              K_local, V_local, L, Hkv, q_offset, scale);
    if (s != MSA_OK) return s;
    const size_t need = msa::attn_workspace(dt, B, Tq, Hq, Hkv, ctx->head_dim, max_rows_per_query, L,
                                            ctx->num_cus);
    if (need > MSA_NOALLOC_SCRATCH_BYTES)
        return fail(MSA_ERR_WORKSPACE,
                    "%s: this call needs %zu bytes of scratch, the library's array holds %zu; "
                    "use msa_sparse_attn with a workspace", fn, need, size_t(MSA_NOALLOC_SCRATCH_BYTES));
    return sparse_attn_fwd(fn, ctx, dt, Q, B, Tq, Hq, KVmem, mem_off, mem_rows_cap, max_rows_per_query, K_local,
                           V_local, L, Hkv, q_offset, scale, O, nullptr, ctx->scratch, MSA_NOALLOC_SCRATCH_BYTES,
                           stream);
}

msa_status msa_sparse_attn_lse(msa_ctx* ctx, msa_dtype dt, const void* Q, int64_t B, int Tq, int Hq,
                               const void* KVmem, const int64_t* mem_off, int64_t mem_rows_cap,
                               int64_t max_rows_per_query, const void* K_local, const void* V_local, int L,
                               int Hkv, int q_offset, float scale, void* O, float* lse, void* workspace,
                               size_t ws_bytes, hipStream_t stream) {
    const char* fn = "msa_sparse_attn_lse";
    if (!lse || (reinterpret_cast<uintptr_t>(lse) & 3u))
        return fail(MSA_ERR_INVALID_ARG, "%s: lse must be a non-NULL, 4-byte aligned device pointer", fn);
    return sparse_attn_fwd(fn, ctx, dt, Q, B, Tq, Hq, KVmem, mem_off, mem_rows_cap, max_rows_per_query, K_local,
                           V_local, L, Hkv, q_offset, scale, O, lse, workspace, ws_bytes, stream);
}

size_t msa_sparse_attn_bwd_workspace_size(msa_dtype dt, int64_t B, int Tq, int Hq, int Hkv,
                                          int64_t max_rows_per_query, int L) {
    if (dt != MSA_BF16 || B < 1 || Tq < 1 || Hq < 1 || Hkv < 1 || max_rows_per_query < 0 || L < 1) return 0;
    return msa::attn_bwd_workspace(B, Tq, Hq, Hkv, max_rows_per_query, L);
}

msa_status msa_sparse_attn_bwd(msa_ctx* ctx, msa_dtype dt, const void* Q, int64_t B, int Tq, int Hq,
                               const void* KVmem, const int64_t* mem_off, int64_t mem_rows_cap,
                               int64_t max_rows_per_query, const void* K_local, const void* V_local, int L,
                               int Hkv, int q_offset, float scale, const void* O, const void* dO,
                               const float* lse, void* dQ, void* dKVmem, void* dK_local, void* dV_local,
                               void* workspace, size_t ws_bytes, hipStream_t stream) {
    const char* fn = "msa_sparse_attn_bwd";
    msa_status s = check_attn(fn, ctx, dt, Q, B, Tq, Hq, KVmem, mem_off, mem_rows_cap, max_rows_per_query,
                              K_local, V_local, L, Hkv, q_offset, scale);
    if (s != MSA_OK) return s;
    if (dt != MSA_BF16 || ctx->head_dim != 128)
        return fail(MSA_ERR_UNSUPPORTED, "%s: the backward takes bf16 with head dim 128", fn);
    if (!O || !dO || !lse || !dQ || !dK_local || !dV_local || (mem_rows_cap > 0 && !dKVmem))
        return fail(MSA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned16(O) || !aligned16(dO) || !aligned16(dQ) || !aligned16(dK_local) || !aligned16(dV_local) ||
        (dKVmem && !aligned16(dKVmem)) || (reinterpret_cast<uintptr_t>(lse) & 3u))
        return fail(MSA_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned (lse 4-byte)", fn);
    const size_t need = msa::attn_bwd_workspace(B, Tq, Hq, Hkv, max_rows_per_query, L);
    if (!workspace || !aligned256(workspace) || ws_bytes < need)
        return fail(MSA_ERR_WORKSPACE, "%s: workspace needs %zu bytes, 256-aligned (got %zu)", fn, need,
                    ws_bytes);
    msa::AttnBwdArgs a{};
    a.f = msa::AttnArgs{dt, Q, B, Tq, Hq, Hkv, ctx->head_dim, L, KVmem, mem_off, mem_rows_cap,
                        max_rows_per_query, K_local, V_local, q_offset, scale, const_cast<void*>(O), workspace,
                        ws_bytes, ctx->rope_cs, ctx->max_pos, ctx->num_cus, nullptr};
    a.dO = dO;
    a.lse = lse;
    a.dQ = dQ;
    a.dKVmem = dKVmem;
    a.dK_local = dK_local;
    a.dV_local = dV_local;
    DeviceGuard dg(ctx->device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "msa_sparse_attn_bwd: hipSetDevice");
    hipError_t e = msa::launch_attn_bwd(a, stream);
    if (e != hipSuccess) return hip_fail(e, "msa_sparse_attn_bwd: launch");
    return ok();
}

size_t msa_gather_attn_workspace_size(msa_dtype dt, int64_t B, int Tq, int Hq, int Hkv, int top_k,
                                      int64_t cap_rows, int64_t max_rows_per_query, int L) {
    if (!dtype_ok(dt) || B < 1 || Tq < 1 || Hq < 1 || Hkv < 1 || top_k < 1 || cap_rows < 0 ||
        max_rows_per_query < 0 || L < 1)
        return 0;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess) cus = prop.multiProcessorCount;
    }
    msa::AttnArgs a{dt, nullptr, B, Tq, Hq, Hkv, 128, L, nullptr, nullptr, cap_rows, max_rows_per_query,
                    nullptr, nullptr, 0, 1.f, nullptr, nullptr, 0, nullptr, 0, cus, nullptr};
    return msa::gather_attn_workspace(a, cap_rows);
}

msa_status msa_gather_attn(msa_ctx* ctx, msa_dtype dt, const void* host_KVbar, size_t row_bytes,
                           int64_t n_rows_host, const int64_t* doc_chunk_off, int64_t n_docs, const int32_t* ids,
                           int top_k, void* dst_KVmem, int64_t cap_rows, int64_t* mem_off, const void* Q, int64_t B,
                           int Tq, int Hq, int64_t max_rows_per_query, const void* K_local, const void* V_local,
                           int L, int Hkv, int q_offset, float scale, void* O, void* workspace, size_t ws_bytes,
                           hipStream_t stream) {
    const char* fn = "msa_gather_attn";
    msa_status s = check_gather_device(fn, ctx, host_KVbar, row_bytes, n_rows_host, doc_chunk_off, n_docs, ids, B,
                                       top_k, dst_KVmem, cap_rows, mem_off);
    if (s != MSA_OK) return s;
    s = check_attn(fn, ctx, dt, Q, B, Tq, Hq, dst_KVmem, mem_off, cap_rows, max_rows_per_query, K_local, V_local,
                   L, Hkv, q_offset, scale);
    if (s != MSA_OK) return s;
    if (row_bytes != size_t(2) * Hkv * ctx->head_dim * dtype_bytes(dt))
        return fail(MSA_ERR_INVALID_ARG, "%s: row_bytes %zu is not one K̄ and one V̄ row (2 x %d x %d x %zu)", fn,
                    row_bytes, Hkv, ctx->head_dim, dtype_bytes(dt));
    if (!O || !aligned16(O)) return fail(MSA_ERR_INVALID_ARG, "%s: O must be a 16-byte aligned pointer", fn);
    msa::GatherAttnArgs ga{msa::AttnArgs{dt, Q, B, Tq, Hq, Hkv, ctx->head_dim, L, dst_KVmem, mem_off, cap_rows,
                                         max_rows_per_query, K_local, V_local, q_offset, scale, O, workspace,
                                         ws_bytes, ctx->rope_cs, ctx->max_pos, ctx->num_cus, nullptr},
                           dst_KVmem, mem_off, host_KVbar, row_bytes, n_rows_host, doc_chunk_off, n_docs, ids,
                           top_k, cap_rows};
    const size_t need = msa::gather_attn_workspace(ga.a, cap_rows);
    if (!workspace || !aligned256(workspace) || ws_bytes < need)
        return fail(MSA_ERR_WORKSPACE, "%s: workspace needs %zu bytes, 256-aligned (got %zu)", fn, need,
                    ws_bytes);
    DeviceGuard dg(ctx->device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "msa_gather_attn: hipSetDevice");
    const hipError_t e = msa::launch_gather_attn(ga, stream);
    if (e != hipSuccess) return hip_fail(e, "msa_gather_attn: launch");
    return ok();
}

}  // extern "C"
