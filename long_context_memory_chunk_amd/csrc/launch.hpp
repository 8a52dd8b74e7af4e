// Internal launchers (not part of the C ABI).  Each returns the HIP error of
// its launches; argument validation happens in api.hip before these run.
#pragma once

#include <hip/hip_ext.h>

#include "common.hpp"

namespace msa {

hipError_t launch_encode(const msa_ctx* ctx, msa_dtype dt, const void* K, const void* V,
                         const void* Kr, const int64_t* tok_off, const int64_t* chunk_off,
                         int64_t n_docs, int64_t T_rows, int64_t N, int hkv, int chunk_len,
                         int64_t max_doc_len, void* KVbar, void* Krbar, hipStream_t st);
hipError_t launch_encode_bwd(const msa_ctx* ctx, msa_dtype dt, const void* dKVbar, const void* dKrbar,
                             const int64_t* tok_off, const int64_t* chunk_off, int64_t n_docs, int64_t T_rows,
                             int64_t N, int hkv, int chunk_len, int64_t max_doc_len, void* dK, void* dV,
                             void* dKr, hipStream_t st);

struct RouteArgs {
    msa_dtype dt;
    const void* Qr;
    int64_t B;
    int Tq, Hq, Hkv, D;
    const void* Krbar;
    int64_t N;
    const int64_t* chunk_off;
    int64_t n_docs;
    int top_k;
    int32_t* out_ids;
    float* out_scores;
    float* out_chunk;
    float* out_doc;
    void* ws;
    size_t ws_bytes;
    int num_cus;
    hipEvent_t prof_start, prof_stop;   // recorded around the main chunk-score kernel if set
};

size_t route_workspace(msa_dtype dt, int64_t B, int Tq, int Hq, int Hkv, int D, int64_t N,
                       int64_t n_docs, int top_k, int num_cus);
hipError_t launch_route(const RouteArgs& a, hipStream_t st);

// Backward of the document score (route_bwd.hip).
struct RouteBwdArgs {
    RouteArgs r;            // Qr, B, Tq, Hq, Hkv, D, Krbar, N, chunk_off, n_docs, dt, ws
    const float* dscore;    // [B][n_docs]
    float* dQr;             // [B][Tq][Hq][D]
    float* dKr;             // [N][Hkv][D]
    void* arg_out;          // optional int32 [B][n_docs][2]: (chunk, token) of each arg max, -1 if none
};
size_t route_bwd_workspace(int64_t B, int Tq, int Hq, int Hkv, int D, int64_t N, int64_t n_docs);
hipError_t launch_route_bwd(const RouteBwdArgs& a, hipStream_t st);

// Records an optional profiling event (NULL: nothing to do).
inline hipError_t record_if(hipEvent_t e, hipStream_t st) {
    return e ? hipEventRecord(e, st) : hipSuccess;
}

// Launches a kernel with optional profiling events that the dispatch itself
// records at the kernel's start and end (both NULL: a plain launch), so timing
// a kernel puts no extra packet, and no gap, between it and its neighbours.
template <typename F, typename... Args>
hipError_t launch_timed(F kernel, dim3 grid, dim3 block, hipStream_t st, hipEvent_t start, hipEvent_t stop,
                        Args... args) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, start, stop, 0, args...);
    return hipGetLastError();
}

struct AttnArgs {
    msa_dtype dt;
    const void* Q;
    int64_t B;
    int Tq, Hq, Hkv, D, L;
    const void* KVmem;
    const int64_t* mem_off;
    int64_t mem_rows_cap, max_rows;
    const void* K_local;
    const void* V_local;
    int q_offset;
    float scale;
    void* O;
    void* ws;
    size_t ws_bytes;
    const float2* rope_cs;
    int max_pos;
    int num_cus;
    float* lse = nullptr;   // optional [B][Tq][Hq]: natural-log log-sum-exp of each row's scaled logits
};

// Memory rows of query b: mem_off[b] .. mem_off[b+1]-1 clamped to [0, cap] and
// to max_rows rows.
__device__ __forceinline__ void mem_range(const int64_t* __restrict__ mem_off, int64_t b, int64_t cap,
                                          int64_t max_rows, int64_t& r0, int64_t& M) {
    int64_t a = mem_off[b], e = mem_off[b + 1];
    a = a < 0 ? 0 : (a > cap ? cap : a);
    e = e < a ? a : (e > cap ? cap : e);
    if (e - a > max_rows) e = a + max_rows;
    r0 = a;
    M = e - a;
}

// Backward of the attention (attn_bwd.hip): bf16, d = 128.
struct AttnBwdArgs {
    AttnArgs f;             // the forward's arguments (O read, not written; ws is the backward's)
    const void* dO;         // [B][Tq][Hq][d]
    const float* lse;       // [B][Tq][Hq], as the forward saved it
    void* dQ;               // [B][Tq][Hq][d]
    void* dKVmem;           // [mem_rows_cap][2][Hkv][d]: rows of each query's memory written
    void* dK_local;         // [B][L][Hkv][d]
    void* dV_local;
};
size_t attn_bwd_workspace(int64_t B, int Tq, int Hq, int Hkv, int64_t max_rows, int L);
hipError_t launch_attn_bwd(const AttnBwdArgs& a, hipStream_t st);

constexpr int kMaxGatherB = 1024;
size_t gather_device_workspace(int64_t B, int64_t cap_rows);
// The copy plan of the device gather (one workgroup): mem_off and, in the
// workspace, the source row of every destination row (*src_of_row).
hipError_t launch_gather_plan(const int32_t* ids, int64_t B, int K, const int64_t* off, int64_t n_docs,
                              int64_t n_rows_host, int64_t cap_rows, int64_t* mem_off, void* ws,
                              int64_t** src_of_row, hipStream_t st);

// The device gather's copy as the gather + local-attention launch runs it:
// the one-query copy (it plans itself from ids and off, and writes mem_off)
// or the bounded copy of a plan (src_of_row; mem_off[B] rows in all).
struct GatherCopyArgs {
    const u32x4* host;
    int64_t row_vecs;
    const int64_t* src_of_row;
    int B;
    const int32_t* ids;
    int K;
    const int64_t* off;
    int64_t n_docs, n_rows_host, cap;
    int64_t* mem_off;
    u32x4* dst;
};
hipError_t launch_gather_device(const void* host, size_t row_bytes, int64_t n_rows_host, const int64_t* off,
                                int64_t n_docs, const int32_t* ids, int64_t B, int K, void* dst,
                                int64_t cap_rows, int64_t* mem_off, void* ws, hipStream_t st);

size_t attn_workspace(msa_dtype dt, int64_t B, int Tq, int Hq, int Hkv, int D,
                      int64_t max_rows, int L, int num_cus);
hipError_t launch_attn(const AttnArgs& a, hipStream_t st);

// The device gather followed by the attention over its rows: dst (cap_rows
// rows) and mem_off are the gather's outputs, which the attention then reads
// (a.KVmem == dst, a.mem_off == mem_off); a.ws is the workspace of
// gather_attn_workspace bytes.
struct GatherAttnArgs {
    AttnArgs a;
    void* dst;
    int64_t* mem_off;
    const void* host;
    size_t row_bytes;
    int64_t n_rows_host;
    const int64_t* off;
    int64_t n_docs;
    const int32_t* ids;
    int K;
    int64_t cap_rows;
};
size_t gather_attn_workspace(const AttnArgs& a, int64_t cap_rows);
hipError_t launch_gather_attn(const GatherAttnArgs& ga, hipStream_t st);

}  // namespace msa
