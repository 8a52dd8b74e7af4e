// Stage 2b, device-side variant: assemble the selected documents' pooled
// K̄/V̄ rows by reading the pinned host store directly from the GPU.
//
// Source: news.neo-ai.one MSA article, 推論パイプライン (Fig. 3): only the
// selected K̄/V̄ are loaded and concatenated with the local context; content
// K̄/V̄ stay in host memory and are fetched when selected.
// ruixiangma.github.io blog, Memory Parallel (CPU-offloaded K̄/V̄ fetched on
// demand).
//
// The layout is the one msa_gather produces (ids of a query in ascending
// order, rows back to back, mem_off prefix sums), but nothing goes through
// the host: the plan (gather_plan_par_kernel, one workgroup per query, or
// gather_plan_kernel past kParPlanB queries) turns the device-resident ids
// into mem_off and a table holding, for every destination row, its source
// row in the host store; gather_copy then reads the host rows over PCIe with 16-byte loads
// (pinned host memory is mapped into the GPU's address space) and writes them
// to HBM.  gather_copy runs on a fixed grid of kCopyWgs workgroups, each with
// kCopyRows rows (32 KB) in flight, which keeps PCIe busy (about 2 MB in
// flight in all) while most CUs stay free for other work, e.g. attention over
// rows gathered earlier, on another stream.  For a single query, gather_one
// does both in one launch: every workgroup sorts the query's K ids and scans
// their row counts itself (a few hundred bytes) and then copies its share.
// No host synchronisation is needed between routing and attention.
#include "common.hpp"
#include "gather_body.hpp"
#include "launch.hpp"

namespace msa {
namespace {

constexpr int kPlanWaves = 16;

__global__ __launch_bounds__(kPlanWaves * 64) void gather_plan_kernel(
    const int32_t* __restrict__ ids, int B, int K, const int64_t* __restrict__ off, int64_t n_docs,
    int64_t n_rows_host, int64_t cap, int64_t* __restrict__ mem_off, int64_t* __restrict__ plan,
    int64_t* __restrict__ src_of_row) {
    __shared__ int64_t totals[kMaxGatherB + 1];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    // a wave's first kRegIters queries keep their plan entries in registers
    // between the phases; later ones (B > 64) go through the plan array
    constexpr int kRegIters = 4;
    int64_t r_src[kRegIters], r_local[kRegIters], r_rows[kRegIters];
    // phase 1: per query, sorted ids, row counts, local prefix
    for (int it = 0, b = wave; b < B; ++it, b += kPlanWaves) {
        int32_t id = (lane < K) ? ids[int64_t(b) * K + lane] : 0x7FFFFFFF;
        if (id < 0 || id >= n_docs) id = 0x7FFFFFFF;          // invalid ids copy nothing
        // bitonic sort, ascending across lanes
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
        const int64_t local = wave_excl_scan(rows, lane);
        if (it < kRegIters) {
#pragma unroll
            for (int u = 0; u < kRegIters; ++u)
                if (u == it) { r_src[u] = src; r_local[u] = local; r_rows[u] = rows; }
        } else {
            int64_t* pb = plan + (int64_t(b) * 64 + lane) * 3;
            pb[0] = src;
            pb[1] = local;
            pb[2] = rows;
        }
        const int64_t tot = lane64(local + rows, 63);
        if (lane == 0) totals[b] = tot;
    }
    __syncthreads();
    // phase 2: query offsets (B is small; one thread)
    if (threadIdx.x == 0) {
        int64_t acc = 0;
        for (int b = 0; b < B; ++b) {
            const int64_t t = totals[b];
            mem_off[b] = acc < cap ? acc : cap;
            totals[b] = acc;
            acc += t;
        }
        mem_off[B] = acc < cap ? acc : cap;
    }
    __syncthreads();
    // phase 3: absolute destination rows, clamped to the buffer, and the
    // source row of every destination row
    for (int it = 0, b = wave; b < B; ++it, b += kPlanWaves) {
        int64_t src = 0, local = 0, rows = 0;
        if (it < kRegIters) {
#pragma unroll
            for (int u = 0; u < kRegIters; ++u)
                if (u == it) { src = r_src[u]; local = r_local[u]; rows = r_rows[u]; }
        } else {
            const int64_t* pb = plan + (int64_t(b) * 64 + lane) * 3;
            src = pb[0];
            local = pb[1];
            rows = pb[2];
        }
        const int64_t dst = local + totals[b];
        if (dst >= cap) rows = 0;
        else if (dst + rows > cap) rows = cap - dst;
        for (int e = 0; e < K; ++e) {
            const int64_t s_e = lane64(src, e), d_e = lane64(dst, e), n_e = lane64(rows, e);
            for (int64_t r = lane; r < n_e; r += kWave) src_of_row[d_e + r] = s_e + r;
        }
    }
}

// The same plan with one workgroup per query, for up to kParPlanB queries:
// wave 0 sorts its query's ids and scans their row counts, while waves 1-3 sum
// the rows of every earlier query's documents (order does not matter for the
// sum) to find where the query's rows start; then the query's source rows are
// written.  Two dependent global reads (ids, then offsets) instead of the
// single workgroup's walk over the queries.  Same results as gather_plan_kernel.
constexpr int kParPlanB = 64;

__global__ __launch_bounds__(256) void gather_plan_par_kernel(
    const int32_t* __restrict__ ids, int B, int K, const int64_t* __restrict__ off, int64_t n_docs,
    int64_t n_rows_host, int64_t cap, int64_t* __restrict__ mem_off, int64_t* __restrict__ src_of_row) {
    __shared__ int64_t s_part[4];
    __shared__ int64_t s_tot;
    const int b = int(blockIdx.x);
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    // rows and first row of document id (none for an invalid id or range);
    // the loads are unconditional (a clamped index) so that several are in
    // flight together
    auto doc_rows = [&](int32_t id, int64_t& src) -> int64_t {
        const bool ok = id >= 0 && id < n_docs;
        const int64_t a = off[ok ? id : 0], e = off[ok ? id + 1 : 0];
        const bool good = ok && a >= 0 && e >= a && e <= n_rows_host;
        src = good ? a : 0;
        return good ? e - a : 0;
    };
    int64_t src = 0, rows = 0, local = 0;
    if (wave == 0) {
        int32_t id = (lane < K) ? ids[int64_t(b) * K + lane] : 0x7FFFFFFF;
        if (id < 0 || id >= n_docs) id = 0x7FFFFFFF;
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
        rows = (id != 0x7FFFFFFF) ? doc_rows(id, src) : 0;
        local = wave_excl_scan(rows, lane);
        if (lane == 63) s_tot = local + rows;
        s_part[0] = 0;
    } else {
        constexpr int kBatch = 4;                       // ids per thread per round trip
        const int64_t n = int64_t(b) * K;
        int64_t acc = 0;
        for (int64_t j0 = threadIdx.x - kWave; j0 < n; j0 += int64_t(3 * kWave) * kBatch) {
            int32_t idv[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int64_t j = j0 + int64_t(u) * 3 * kWave;
                idv[u] = j < n ? ids[j] : -1;
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                int64_t unused;
                acc += doc_rows(idv[u], unused);
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
        if (lane == 0) s_part[wave] = acc;
    }
    __syncthreads();
    const int64_t base = s_part[1] + s_part[2] + s_part[3];
    if (threadIdx.x == 0) {
        mem_off[b] = base < cap ? base : cap;
        if (b == B - 1) mem_off[B] = base + s_tot < cap ? base + s_tot : cap;
    }
    if (wave == 0) {
        const int64_t dst = local + base;
        if (dst >= cap) rows = 0;
        else if (dst + rows > cap) rows = cap - dst;
        for (int e = 0; e < K; ++e) {
            const int64_t s_e = lane64(src, e), d_e = lane64(dst, e), n_e = lane64(rows, e);
            for (int64_t r = lane; r < n_e; r += kWave) src_of_row[d_e + r] = s_e + r;
        }
    }
}

__global__ __launch_bounds__(256) void gather_copy_kernel(const u32x4* __restrict__ host, int64_t row_vecs,
                                                          const int64_t* __restrict__ src_of_row,
                                                          const int64_t* __restrict__ mem_off, int B,
                                                          u32x4* __restrict__ dst) {
    gather_copy_wg(host, row_vecs, src_of_row, mem_off, B, dst, int(blockIdx.x), kCopyWgs);
}

// gather_one: every selected row is requested at once, whatever the
// document sizes (kOneRows rows per workgroup, all in flight together).
__global__ __launch_bounds__(256) void gather_one_kernel(const u32x4* __restrict__ host, int64_t row_vecs,
                                                         const int32_t* __restrict__ ids, int K,
                                                         const int64_t* __restrict__ off, int64_t n_docs,
                                                         int64_t n_rows_host, int64_t cap, int64_t* __restrict__ mem_off,
                                                         u32x4* __restrict__ dst) {
    gather_one_wg(host, row_vecs, ids, K, off, n_docs, n_rows_host, cap, mem_off, dst, int(blockIdx.x));
}

}  // namespace

size_t gather_device_workspace(int64_t B, int64_t cap_rows) {
    return align256(size_t(B) * 64 * 3 * sizeof(int64_t)) + align256(size_t(cap_rows) * sizeof(int64_t));
}

hipError_t launch_gather_plan(const int32_t* ids, int64_t B, int K, const int64_t* off, int64_t n_docs,
                              int64_t n_rows_host, int64_t cap_rows, int64_t* mem_off, void* ws,
                              int64_t** src_of_row, hipStream_t st) {
    int64_t* plan = static_cast<int64_t*>(ws);
    *src_of_row = reinterpret_cast<int64_t*>(static_cast<char*>(ws) + align256(size_t(B) * 64 * 3 * 8));
    if (B <= kParPlanB)
        hipLaunchKernelGGL(gather_plan_par_kernel, dim3(unsigned(B)), dim3(256), 0, st, ids, int(B), K, off, n_docs,
                           n_rows_host, cap_rows, mem_off, *src_of_row);
    else
        hipLaunchKernelGGL(gather_plan_kernel, dim3(1), dim3(kPlanWaves * 64), 0, st, ids, int(B), K, off, n_docs,
                           n_rows_host, cap_rows, mem_off, plan, *src_of_row);
    return hipGetLastError();
}

hipError_t launch_gather_device(const void* host, size_t row_bytes, int64_t n_rows_host, const int64_t* off,
                                int64_t n_docs, const int32_t* ids, int64_t B, int K, void* dst,
                                int64_t cap_rows, int64_t* mem_off, void* ws, hipStream_t st) {
    if (B == 1 && cap_rows <= kOneMaxRows) {
        const int64_t wgs = ceil_div(cap_rows, int64_t(kOneRows));
        hipLaunchKernelGGL(gather_one_kernel, dim3(unsigned(wgs > 0 ? wgs : 1)), dim3(256), 0, st,
                           static_cast<const u32x4*>(host), int64_t(row_bytes / 16), ids, K, off, n_docs,
                           n_rows_host, cap_rows, mem_off, static_cast<u32x4*>(dst));
        return hipGetLastError();
    }
    int64_t* src_of_row = nullptr;
    hipError_t err = launch_gather_plan(ids, B, K, off, n_docs, n_rows_host, cap_rows, mem_off, ws, &src_of_row, st);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(gather_copy_kernel, dim3(kCopyWgs), dim3(256), 0, st, static_cast<const u32x4*>(host),
                       int64_t(row_bytes / 16), src_of_row, mem_off, int(B), static_cast<u32x4*>(dst));
    return hipGetLastError();
}

}  // namespace msa
