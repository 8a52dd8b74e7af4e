// Shared device/host helpers of the MSA library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/msa.h"

namespace msa {

constexpr int kWave = 64;

// ---------------------------------------------------------------- dtypes

struct bf16_t { uint16_t bits; };

// Native 16-byte vector (usable with the nontemporal builtins).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return uint16_t((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

// Two floats -> packed bf16 bits (a in the low half) on the hardware
// converter, which rounds to nearest even like f32_to_bf16.
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2_hw v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Load/store of a scalar element of either storage type as float.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kBytes = 4;
    __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
    static constexpr int kBytes = 2;
    __device__ __forceinline__ static float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i].bits); }
    __device__ __forceinline__ static void store(bf16_t* p, int64_t i, float v) { p[i].bits = f32_to_bf16(v); }
};

// 16-byte vector of either type, unpacked to floats.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
    static constexpr int kN = 4;
    __device__ __forceinline__ static void load(const float* p, float* out) {
        float4 v = *reinterpret_cast<const float4*>(p);
        out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
    }
    __device__ __forceinline__ static void store(float* p, const float* in) {
        *reinterpret_cast<float4*>(p) = make_float4(in[0], in[1], in[2], in[3]);
    }
};
template <> struct Vec16<bf16_t> {
    static constexpr int kN = 8;
    __device__ __forceinline__ static void load(const bf16_t* p, float* out) {
        uint4 v = *reinterpret_cast<const uint4*>(p);
        out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x);
        out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
        out[4] = bf16_lo(v.z); out[5] = bf16_hi(v.z);
        out[6] = bf16_lo(v.w); out[7] = bf16_hi(v.w);
    }
    __device__ __forceinline__ static void store(bf16_t* p, const float* in) {
        uint4 v;
        v.x = uint32_t(f32_to_bf16(in[0])) | (uint32_t(f32_to_bf16(in[1])) << 16);
        v.y = uint32_t(f32_to_bf16(in[2])) | (uint32_t(f32_to_bf16(in[3])) << 16);
        v.z = uint32_t(f32_to_bf16(in[4])) | (uint32_t(f32_to_bf16(in[5])) << 16);
        v.w = uint32_t(f32_to_bf16(in[6])) | (uint32_t(f32_to_bf16(in[7])) << 16);
        *reinterpret_cast<uint4*>(p) = v;
    }
};

// ---------------------------------------------------------------- DPP

// DPP controls (GFX9 encoding).
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

template <int Ctrl>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, 0xF, 0xF, false));
}

// Sum over aligned groups of Lanes consecutive lanes (Lanes in {1,2,4,8,16,32,64});
// every lane of a group receives the group's sum.
template <int Lanes>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (Lanes >= 2) v += dpp<kQuadXor1>(v);
    if constexpr (Lanes >= 4) v += dpp<kQuadXor2>(v);
    if constexpr (Lanes >= 8) v += dpp<kRowHalfMirror>(v);
    if constexpr (Lanes >= 16) v += dpp<kRowMirror>(v);
    if constexpr (Lanes >= 32) v += __shfl_xor(v, 16);
    if constexpr (Lanes >= 64) v += __shfl_xor(v, 32);
    return v;
}

template <int Lanes>
__device__ __forceinline__ float group_max(float v) {
    if constexpr (Lanes >= 2) v = fmaxf(v, dpp<kQuadXor1>(v));
    if constexpr (Lanes >= 4) v = fmaxf(v, dpp<kQuadXor2>(v));
    if constexpr (Lanes >= 8) v = fmaxf(v, dpp<kRowHalfMirror>(v));
    if constexpr (Lanes >= 16) v = fmaxf(v, dpp<kRowMirror>(v));
    if constexpr (Lanes >= 32) v = fmaxf(v, __shfl_xor(v, 16));
    if constexpr (Lanes >= 64) v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }
__device__ __forceinline__ float wave_max(float v) { return group_max<64>(v); }

// ---------------------------------------------------------------- launch plumbing

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace msa

// The context shared by the host side and the launchers.
struct msa_ctx {
    int device;
    int head_dim;
    double theta;
    int max_pos;
    int num_cus;
    float2* rope_cs;   // device [max_pos][head_dim/2] (cos, sin)
    hipEvent_t prof_start;   // msa_route_time_next: consumed by the next msa_route
    hipEvent_t prof_stop;
    void* scratch;           // device address of this device's library scratch array
};
