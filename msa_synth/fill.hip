// Device fill for the counter-based synthetic generator (input generation
// only; no part of the method), and a plain streaming-read probe that
// measures what this HBM delivers to a read-only kernel (measurement only).  Element i of stream s under seed is
// SplitMix64 output number i+1 from the state key(seed, s) (Steele, Lea and
// Flood, OOPSLA 2014); four 6-bit fields of it are summed, centred and divided
// by 32, which is exact in bfloat16.  Bit-identical to msa_synth/gen.py.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__host__ __device__ inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

__host__ __device__ inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
    return mix64(mix64(seed) ^ (stream * 0xD1B54A32D192ED03ULL));
}

__device__ inline uint16_t counter_bf16(uint64_t key, uint64_t idx) {
    const uint64_t z = mix64(key + (idx + 1) * 0x9E3779B97F4A7C15ULL);
    const int s = int(z & 63) + int((z >> 6) & 63) + int((z >> 12) & 63) + int((z >> 18) & 63);
    const float f = float(s - 126) / 32.0f;      // exact
    return uint16_t(__float_as_uint(f) >> 16);   // exact truncation of an exact value
}

// dst[k] = element (start + k), k < count; 8 elements per thread, 16-byte stores.
__global__ __launch_bounds__(256) void fill_counter_bf16(uint16_t* __restrict__ dst, uint64_t key,
                                                         uint64_t start, uint64_t count) {
    const uint64_t n8 = count / 8;
    const uint64_t stride = uint64_t(gridDim.x) * 256;
    for (uint64_t v = uint64_t(blockIdx.x) * 256 + threadIdx.x; v < n8; v += stride) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint64_t i = start + v * 8 + 2 * k;
            w[k] = uint32_t(counter_bf16(key, i)) | (uint32_t(counter_bf16(key, i + 1)) << 16);
        }
        reinterpret_cast<uint4*>(dst)[v] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    const uint64_t t = uint64_t(blockIdx.x) * 256 + threadIdx.x;
    if (t < count - n8 * 8) dst[n8 * 8 + t] = counter_bf16(key, start + n8 * 8 + t);
}

// Streaming read of n16 16-byte units: each wave keeps 16 non-temporal 1 KB
// wave loads in flight, batches of 16 consecutive KB dealt grid-strided over
// the waves; the XOR of everything a lane read goes to sink so the loads are
// not optimised away.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_probe(const u32x4_t* __restrict__ src, uint64_t n16,
                                                  uint32_t* __restrict__ sink) {
    constexpr int kLoads = 16;
    const int lane = threadIdx.x % 64;
    const uint64_t wave = uint64_t(blockIdx.x) * 4 + threadIdx.x / 64;
    const uint64_t n_waves = uint64_t(gridDim.x) * 4;
    const uint64_t batches = (n16 + 64 * kLoads - 1) / (64 * kLoads);
    uint32_t acc = 0;
    for (uint64_t b = wave; b < batches; b += n_waves) {
        u32x4_t x[kLoads];
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            const uint64_t i = (b * kLoads + k) * 64 + lane;
            x[k] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < kLoads; ++k) acc ^= x[k].x ^ x[k].y ^ x[k].z ^ x[k].w;
    }
    sink[wave * 64 + lane] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from device memory `src` with `blocks`
// workgroups of 4 waves; sink holds blocks * 256 uint32 (device memory).
int msa_synth_read_probe(const void* src, uint64_t bytes, uint32_t* sink, int blocks, hipStream_t st) {
    if (!src || !sink || blocks < 1 || (bytes & 15u) || (reinterpret_cast<uintptr_t>(src) & 15u))
        return int(hipErrorInvalidValue);
    hipLaunchKernelGGL(read_probe, dim3(unsigned(blocks)), dim3(256), 0, st, static_cast<const u32x4_t*>(src),
                       bytes / 16, sink);
    return int(hipGetLastError());
}

// Fills dst[0 .. count) (device or pinned host memory, 16-byte aligned) with
// elements start .. start+count-1 of stream `stream` under `seed`, as bf16 bits.
int msa_synth_fill_counter_bf16(void* dst, uint64_t seed, uint64_t stream, uint64_t start,
                                uint64_t count, hipStream_t st) {
    if (count == 0) return 0;
    if (!dst || (reinterpret_cast<uintptr_t>(dst) & 15u)) return int(hipErrorInvalidValue);
    uint64_t blocks = (count / 8 + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(fill_counter_bf16, dim3(unsigned(blocks)), dim3(256), 0, st,
                       static_cast<uint16_t*>(dst), stream_key(seed, stream), start, count);
    return int(hipGetLastError());
}

uint64_t msa_synth_stream_key(uint64_t seed, uint64_t stream) { return stream_key(seed, stream); }

}  // extern "C"
