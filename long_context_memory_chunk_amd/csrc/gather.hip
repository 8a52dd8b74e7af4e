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
// the host: gather_plan turns the device-resident ids into (source row,
// destination row, rows) triples, and gather_copy reads the host rows over
// PCIe with 16-byte loads (pinned host memory is mapped into the GPU's
// address space) and writes them to HBM.  No host synchronisation is needed
// between routing and attention.
#include "common.hpp"
#include "launch.hpp"

namespace msa {
namespace {

constexpr int kPlanWaves = 16;

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

__global__ __launch_bounds__(kPlanWaves * 64) void gather_plan_kernel(
    const int32_t* __restrict__ ids, int B, int K, const int64_t* __restrict__ off, int64_t n_docs,
    int64_t n_rows_host, int64_t cap, int64_t* __restrict__ mem_off, int64_t* __restrict__ plan) {
    __shared__ int64_t totals[kMaxGatherB + 1];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    // phase 1: per query, sorted ids, row counts, local prefix
    for (int b = wave; b < B; b += kPlanWaves) {
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
        int64_t* pb = plan + (int64_t(b) * 64 + lane) * 3;
        pb[0] = src;
        pb[1] = local;
        pb[2] = rows;
        const int64_t tot = __shfl(local + rows, 63);
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
    // phase 3: absolute destination rows, clamped to the buffer
    for (int b = wave; b < B; b += kPlanWaves) {
        int64_t* pb = plan + (int64_t(b) * 64 + lane) * 3;
        int64_t dst = pb[1] + totals[b];
        int64_t rows = pb[2];
        if (dst >= cap) rows = 0;
        else if (dst + rows > cap) rows = cap - dst;
        pb[1] = dst;
        pb[2] = rows;
    }
}

// grid (B * 64 plan entries, kCopySplit); workgroup y copies rows y, y + kCopySplit, ...
constexpr int kCopySplit = 8;

__global__ __launch_bounds__(256) void gather_copy_kernel(const u32x4* __restrict__ host, int64_t row_vecs,
                                                          const int64_t* __restrict__ plan, int K,
                                                          u32x4* __restrict__ dst) {
    const int64_t e = blockIdx.x;
    if (int(e % 64) >= K) return;
    const int64_t src_row = plan[e * 3], dst_row = plan[e * 3 + 1], rows = plan[e * 3 + 2];
    for (int64_t r = blockIdx.y; r < rows; r += kCopySplit) {
        const u32x4* s = host + (src_row + r) * row_vecs;
        u32x4* d = dst + (dst_row + r) * row_vecs;
        for (int64_t v = threadIdx.x; v < row_vecs; v += 256) d[v] = s[v];
    }
}

}  // namespace

size_t gather_device_workspace(int64_t B) { return align256(size_t(B) * 64 * 3 * sizeof(int64_t)); }

hipError_t launch_gather_device(const void* host, size_t row_bytes, int64_t n_rows_host, const int64_t* off,
                                int64_t n_docs, const int32_t* ids, int64_t B, int K, void* dst,
                                int64_t cap_rows, int64_t* mem_off, void* ws, hipStream_t st) {
    int64_t* plan = static_cast<int64_t*>(ws);
    hipLaunchKernelGGL(gather_plan_kernel, dim3(1), dim3(kPlanWaves * 64), 0, st, ids, int(B), K, off, n_docs,
                       n_rows_host, cap_rows, mem_off, plan);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(gather_copy_kernel, dim3(unsigned(B * 64), kCopySplit), dim3(256), 0, st,
                       static_cast<const u32x4*>(host), int64_t(row_bytes / 16), plan, K,
                       static_cast<u32x4*>(dst));
    return hipGetLastError();
}

}  // namespace msa
