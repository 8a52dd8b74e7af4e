// Workgroup bodies of the device-side gather (stage 2b), shared by the gather
// kernels (gather.hip) and by the launch that runs the copy beside the
// attention over the local keys (attn_decode_mfma.hip).
//
// Source: news.neo-ai.one MSA article, 推論パイプライン (Fig. 3): only the
// selected K̄/V̄ are loaded from host memory and concatenated with the local
// context; ruixiangma.github.io blog, Memory Parallel (CPU-offloaded K̄/V̄
// fetched on demand).
#pragma once

#include "common.hpp"

namespace msa {

// Bounded copy: destination rows are dealt to n_wgs workgroups kCopyRows at a
// time (rows w * kCopyRows + j, then + n_wgs * kCopyRows, ...); a thread
// copies one 16-byte unit of each of its workgroup's kCopyRows rows, all
// loads issued before the stores.
constexpr int kCopyWgs = 64;
constexpr int kCopyRows = 8;
// One-query copy: workgroup w copies destination rows w * kOneRows .. + kOneRows - 1.
constexpr int kOneRows = 2;
constexpr int64_t kOneMaxRows = 8192;   // larger capacities take the plan + bounded copy path
// One-query copy that also attends over the rows it copies (a one-token
// query, KV heads <= 8): destination rows per workgroup, 4 while the
// partials (one per workgroup) fit the combine, else 8.
constexpr int kOneAttnRowsFew = 4;
constexpr int kOneAttnRowsMany = 8;

// Lane `src` of a 64-bit value, for a wave-uniform lane index (two scalar
// reads instead of two LDS permutes).
__device__ __forceinline__ int64_t lane64(int64_t v, int src) {
    const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v)), src));
    const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(uint64_t(v) >> 32)), src));
    return int64_t((uint64_t(hi) << 32) | lo);
}

__device__ __forceinline__ int64_t wave_excl_scan(int64_t v, int lane) {
    // inclusive Hillis-Steele scan over 64 lanes, then shift to exclusive
    int64_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    return x - v;
}

// Bounded copy by workgroup wg of n_wgs (256 threads): src_of_row and
// mem_off[B] (the number of destination rows) come from gather_plan.
__device__ __forceinline__ void gather_copy_wg(const u32x4* __restrict__ host, int64_t row_vecs,
                                               const int64_t* __restrict__ src_of_row,
                                               const int64_t* __restrict__ mem_off, int B,
                                               u32x4* __restrict__ dst, int wg, int n_wgs) {
    const int64_t total = mem_off[B];
    const int64_t stride = int64_t(n_wgs) * kCopyRows;
    int64_t src[kCopyRows];
    int64_t r0 = int64_t(wg) * kCopyRows;
#pragma unroll
    for (int j = 0; j < kCopyRows; ++j) src[j] = (r0 + j < total) ? src_of_row[r0 + j] : -1;
    for (; r0 < total; r0 += stride) {
        // the next round's source rows are read while this round's first
        // units come over PCIe, so a round waits on no HBM read of its own
        // (every thread takes the first pass, row_vecs >= 1; units past the
        // row are skipped, not broken out of)
        int64_t nxt[kCopyRows];
        for (int64_t v0 = 0; v0 < row_vecs; v0 += 256) {
            const int64_t v = v0 + threadIdx.x;
            const bool on = v < row_vecs;
            u32x4 x[kCopyRows];
#pragma unroll
            for (int j = 0; j < kCopyRows; ++j)
                if (on && src[j] >= 0) x[j] = host[src[j] * row_vecs + v];
            if (v0 == 0) {
#pragma unroll
                for (int j = 0; j < kCopyRows; ++j)
                    nxt[j] = (r0 + stride + j < total) ? src_of_row[r0 + stride + j] : -1;
            }
#pragma unroll
            for (int j = 0; j < kCopyRows; ++j)
                if (on && src[j] >= 0) dst[(r0 + j) * row_vecs + v] = x[j];
        }
#pragma unroll
        for (int j = 0; j < kCopyRows; ++j) src[j] = nxt[j];
    }
}

// One-query plan for destination rows wg * R .. wg * R + R - 1 (256 threads):
// each wave derives it on its own (wave-uniform results, no barrier): the K
// ids sorted, their row counts and prefix sums; a destination row's entry is
// the last one starting at or before it (a ballot).  sr[j] is the source row
// of destination row wg * R + j, or -1 past the end.  Workgroup 0 also writes
// mem_off.  Returns the number of destination rows.
template <int R>
__device__ __forceinline__ int64_t gather_one_plan(const int32_t* __restrict__ ids, int K,
                                                   const int64_t* __restrict__ off, int64_t n_docs,
                                                   int64_t n_rows_host, int64_t cap, int64_t* __restrict__ mem_off,
                                                   int wg, int64_t (&sr)[R]) {
    const int lane = threadIdx.x % kWave;
    int32_t id = (lane < K) ? ids[lane] : 0x7FFFFFFF;
    if (id < 0 || id >= n_docs) id = 0x7FFFFFFF;          // invalid ids copy nothing
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const int32_t y = __shfl_xor(id, j);
            const bool asc_block = (lane & k) == 0;
            const bool lower = (lane & j) == 0;
            const int32_t mn = id < y ? id : y, mx = id < y ? y : id;
            id = (lower == asc_block) ? mn : mx;
        }
    }
    int64_t src = 0, rows = 0;
    if (id != 0x7FFFFFFF) {
        src = off[id];
        const int64_t end = off[id + 1];
        if (src >= 0 && end >= src && end <= n_rows_host) rows = end - src;
        else src = 0;
    }
    const int64_t dst0 = wave_excl_scan(rows, lane);
    int64_t total = lane64(dst0 + rows, 63);
    total = total < cap ? total : cap;
    if (wg == 0 && threadIdx.x == 0) {
        mem_off[0] = 0;
        mem_off[1] = total;
    }
    const int64_t r0 = int64_t(wg) * R;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t r = r0 + j;
        sr[j] = -1;
        if (r < total) {
            // the entry holding destination row r: the last lane with rows and dst0 <= r
            const uint64_t m = __ballot(rows > 0 && dst0 <= r);
            const int e = 63 - __builtin_clzll(m);
            sr[j] = lane64(src, e) + (r - lane64(dst0, e));
        }
    }
    return total;
}

// One-query copy by workgroup wg (256 threads): destination rows wg * kOneRows
// .. + kOneRows - 1, planned by gather_one_plan.
__device__ __forceinline__ void gather_one_wg(const u32x4* __restrict__ host, int64_t row_vecs,
                                              const int32_t* __restrict__ ids, int K,
                                              const int64_t* __restrict__ off, int64_t n_docs,
                                              int64_t n_rows_host, int64_t cap, int64_t* __restrict__ mem_off,
                                              u32x4* __restrict__ dst, int wg) {
    int64_t sr[kOneRows];
    gather_one_plan<kOneRows>(ids, K, off, n_docs, n_rows_host, cap, mem_off, wg, sr);
    const int64_t r0 = int64_t(wg) * kOneRows;
    for (int64_t v0 = 0; v0 < row_vecs; v0 += 256) {
        const int64_t v = v0 + threadIdx.x;
        if (v >= row_vecs) break;
        u32x4 x[kOneRows];
#pragma unroll
        for (int j = 0; j < kOneRows; ++j)
            if (sr[j] >= 0) x[j] = host[sr[j] * row_vecs + v];
#pragma unroll
        for (int j = 0; j < kOneRows; ++j)
            if (sr[j] >= 0) dst[(r0 + j) * row_vecs + v] = x[j];
    }
}

}  // namespace msa
