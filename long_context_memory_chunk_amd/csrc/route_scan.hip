// Stage 2a (online), chunk scores on the vector units: the unit-query group
// sums and the two VALU scans of the pooled routing keys.
//
// Source: news.neo-ai.one MSA article, 全体設計 › アーキテクチャ (Fig. 2):
// relevance is the cosine similarity of Qr with K̄r, averaged over heads and
// then maximised over tokens; 推論パイプライン (Fig. 3): K̄r is matched
// online.  github-eval-reports review, 核心模块 (head mean first, then token
// max).
//
// Group fold (exact in real arithmetic):
//   sum_h cos(q_h, k_{g(h)}) = sum_g (sum_{h in g} q_h/|q_h|) . k_g / |k_g|
// so route_prep builds U[q][g] = sum_{h in g} q_h / max(|q_h|, eps) once per
// call, and each (query, chunk) costs Hkv*d multiply-adds plus one norm per
// chunk head.
//
// Kernels
//   route_prep            U (fp32) from Qr (route_prep_bf16_d128 for bf16 rows of
//                         128: 16-byte loads, one wave load per four heads).
//   route_scan_bf16_d128  decode scan for B*Tq <= 4: streams K̄r with 16-byte
//                         coalesced loads (a 1 KiB wave load per 4 heads), dot
//                         and norm partials per lane, DPP reduction over the
//                         16 lanes of a head, cross-group sum by readlane.
//                         HBM-bound (1 flop per byte at B*Tq = 1).  With a
//                         16-byte aligned Qr every wave forms the U slice it
//                         needs from Qr itself (unit_group_slice, the same
//                         operations in the same order as route_prep_bf16_d128,
//                         so U is bit-identical) and no prep launch precedes it.
//   route_scan_generic    any dtype/shape: one thread per (query, chunk).
#include "common.hpp"
#include "launch.hpp"
#include "route_scan.hpp"

namespace msa {
namespace {

constexpr float kEps = 1e-8f;

// ---------------------------------------------------------------- prep

template <typename T, int D>
__global__ __launch_bounds__(64) void route_prep_kernel(const T* __restrict__ Qr, int Hq, int hkv,
                                                        float* __restrict__ U) {
    constexpr int PER = D / kWave;
    const int64_t q = blockIdx.x / hkv;
    const int g = blockIdx.x % hkv;
    const int G = Hq / hkv;
    const int lane = threadIdx.x;
    float u[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) u[p] = 0.f;
    for (int h = g * G; h < (g + 1) * G; ++h) {
        const int64_t base = (q * Hq + h) * D + lane * PER;
        float x[PER], s = 0.f;
#pragma unroll
        for (int p = 0; p < PER; ++p) { x[p] = Elem<T>::load(Qr, base + p); s += x[p] * x[p]; }
        s = wave_sum(s);
        const float inv = 1.f / fmaxf(sqrtf(s), kEps);
#pragma unroll
        for (int p = 0; p < PER; ++p) u[p] += x[p] * inv;
    }
    const int64_t ob = (q * hkv + g) * D + lane * PER;
#pragma unroll
    for (int p = 0; p < PER; ++p) U[ob + p] = u[p];
}

// bf16 rows of 128: lane l loads the 16-byte slot l % 16 of head l / 16 of a
// batch of four heads (one 1 KB wave load per batch), reduces each head's
// squared norm over its 16 lanes, adds its unit vector into its slot, and the
// four heads' partial sums meet by two shuffles; lanes 0..15 store the group's
// 128 values.  (The per-element form above reads two bytes per lane per load
// instruction and took 38 us on an 8,192-token prompt's 64 MB.)
__global__ __launch_bounds__(256) void route_prep_bf16_d128(const u32x4* __restrict__ Qr, int64_t n_items,
                                                            int Hq, int hkv, float* __restrict__ U) {
    const int G = Hq / hkv;
    const int lane = threadIdx.x % kWave, sub = lane / 16, c = lane % 16;
    for (int64_t it = int64_t(blockIdx.x) * 4 + threadIdx.x / kWave; it < n_items; it += int64_t(gridDim.x) * 4) {
        const int64_t q = it / hkv;
        const int g = int(it % hkv);
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        for (int h0 = g * G; h0 < (g + 1) * G; h0 += 4) {
            const int h = h0 + sub;
            u32x4 w = {0u, 0u, 0u, 0u};
            if (h < (g + 1) * G) w = Qr[(q * Hq + h) * 16 + c];
            float x[8];
            x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
            x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
            float n2 = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) n2 += x[e] * x[e];
            n2 = group_sum<16>(n2);
            const float inv = 1.f / fmaxf(sqrtf(n2), kEps);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += x[e] * inv;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[e] += __shfl_xor(acc[e], 16);
            acc[e] += __shfl_xor(acc[e], 32);
        }
        if (sub == 0) {
            float4* o = reinterpret_cast<float4*>(U + (q * hkv + g) * 128 + c * 8);
            o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
            o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        }
    }
}

// ---------------------------------------------------------------- decode scan

// Elements e0 .. e0+7 of U[q][g] for bf16 rows of 128, formed by one lane from
// Qr with the operations of route_prep_bf16_d128 in its order: the 16 lanes
// that share g each read their 16-byte slot of head h, the head's squared norm
// is summed over those lanes, and the unit values of heads g*G + 4t + s
// (t = 0, 1, ..) gather in a[s] before (a0 + a1) + (a2 + a3), which is the
// order of that kernel's two cross-slot shuffles.  Every lane of a 16-lane
// group must call it with the same q and g (the norm sum crosses them).
__device__ __forceinline__ void unit_group_slice(const u32x4* __restrict__ Qr, int64_t q, int g, int Hq,
                                                 int G, int c, float out[8]) {
    float a[4][8];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) a[s][e] = 0.f;
    for (int h0 = g * G; h0 < (g + 1) * G; h0 += 4) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int h = h0 + s;
            u32x4 w = {0u, 0u, 0u, 0u};
            if (h < (g + 1) * G) w = Qr[(q * Hq + h) * 16 + c];
            float x[8];
            x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
            x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
            float n2 = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) n2 += x[e] * x[e];
            n2 = group_sum<16>(n2);
            const float inv = 1.f / fmaxf(sqrtf(n2), kEps);
#pragma unroll
            for (int e = 0; e < 8; ++e) a[s][e] += x[e] * inv;
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (a[0][e] + a[1][e]) + (a[2][e] + a[3][e]);
}

// Row n of K̄r is hkv*128 bf16 = LPR KiB; wave load j of a row covers heads
// 4j .. 4j+3, 16 lanes per head, 8 elements per lane.
// Fused: U is formed from Qr (16-byte aligned rows of Hq heads) instead of read.
template <int LPR, int NQ, bool Fused>
__global__ __launch_bounds__(256) void route_scan_bf16_d128(
    const u32x4* __restrict__ Kr, int64_t N, const float* __restrict__ U, const u32x4* __restrict__ Qr, int Hq,
    int B, int Tq, float inv_hq, float* __restrict__ cout) {
    // rows in flight per wave: 8 (16 KiB) when registers allow, else 4
    constexpr int UNROLL = (LPR * NQ <= 2) ? 8 : 4;
    const int lane = threadIdx.x % kWave;
    const int64_t wave_id = int64_t(blockIdx.x) * 4 + threadIdx.x / kWave;
    const int64_t n_waves = int64_t(gridDim.x) * 4;
    const int sub = lane / 16;          // head within the wave load
    const int e0 = (lane % 16) * 8;     // first element within the head
    constexpr int HKV = LPR * 4;

    float u[NQ][LPR][8];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int j = 0; j < LPR; ++j) {
            if constexpr (Fused) {
                unit_group_slice(Qr, q, j * 4 + sub, Hq, Hq / HKV, lane % 16, u[q][j]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) u[q][j][e] = U[(int64_t(q) * HKV + j * 4 + sub) * 128 + e0 + e];
            }
        }

    const int64_t n_groups = (N + 63) / 64;
    for (int64_t grp = wave_id; grp < n_groups; grp += n_waves) {
        const int64_t r_base = grp * 64;
        const int rows = int((N - r_base) < 64 ? (N - r_base) : 64);
        float mine[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) mine[q] = 0.f;
        for (int rr = 0; rr < rows; rr += UNROLL) {
            u32x4 x[UNROLL][LPR];
#pragma unroll
            for (int k = 0; k < UNROLL; ++k) {
                const int r = (rr + k < rows) ? rr + k : rows - 1;   // stay in bounds
                const u32x4* p = Kr + (r_base + r) * (LPR * 64) + lane;
#pragma unroll
                for (int j = 0; j < LPR; ++j) x[k][j] = __builtin_nontemporal_load(p + j * 64);
            }
#pragma unroll
            for (int k = 0; k < UNROLL; ++k) {
                float acc[NQ];
#pragma unroll
                for (int q = 0; q < NQ; ++q) acc[q] = 0.f;
#pragma unroll
                for (int j = 0; j < LPR; ++j) {
                    float f[8];
                    f[0] = bf16_lo(x[k][j].x); f[1] = bf16_hi(x[k][j].x);
                    f[2] = bf16_lo(x[k][j].y); f[3] = bf16_hi(x[k][j].y);
                    f[4] = bf16_lo(x[k][j].z); f[5] = bf16_hi(x[k][j].z);
                    f[6] = bf16_lo(x[k][j].w); f[7] = bf16_hi(x[k][j].w);
                    float n2 = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) n2 += f[e] * f[e];
                    n2 = group_sum<16>(n2);
                    // 1 / max(|k|, eps) as one reciprocal square root (1 ulp)
                    const float rn = __builtin_amdgcn_rsqf(fmaxf(n2, kEps * kEps));
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        float dq = 0.f;
#pragma unroll
                        for (int e = 0; e < 8; ++e) dq += u[q][j][e] * f[e];
                        dq = group_sum<16>(dq);
                        acc[q] += dq * rn;
                    }
                }
                float sc[NQ];
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    float t = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc[q]), 0));
                    t += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc[q]), 16));
                    t += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc[q]), 32));
                    t += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc[q]), 48));
                    sc[q] = t * inv_hq;
                }
                if (lane == rr + k) {
#pragma unroll
                    for (int q = 0; q < NQ; ++q) mine[q] = sc[q];
                }
            }
        }
        if (lane < rows) {
            for (int b = 0; b < B; ++b) {
                float m = -INFINITY;
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    if (q / Tq == b) m = fmaxf(m, mine[q]);
                cout[int64_t(b) * N + r_base + lane] = m;
            }
        }
    }
}

// ---------------------------------------------------------------- generic scan

constexpr int kMaxHkvGeneric = 32;

template <typename T, int D>
__global__ __launch_bounds__(256) void route_scan_generic(
    const T* __restrict__ Kr, int64_t N, int hkv, const float* __restrict__ U, int64_t B, int Tq,
    float inv_hq, float* __restrict__ cout) {
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= B * N) return;
    const int64_t b = idx / N, n = idx % N;
    const T* row = Kr + n * hkv * D;
    float rn[kMaxHkvGeneric];
    for (int g = 0; g < hkv; ++g) {
        float s = 0.f;
        for (int i = 0; i < D; ++i) { const float x = Elem<T>::load(row, g * D + i); s += x * x; }
        rn[g] = 1.f / fmaxf(sqrtf(s), kEps);
    }
    float best = -INFINITY;
    for (int t = 0; t < Tq; ++t) {
        const float* uq = U + (b * Tq + t) * hkv * D;
        float tot = 0.f;
        for (int g = 0; g < hkv; ++g) {
            float dq = 0.f;
            for (int i = 0; i < D; ++i) dq += uq[g * D + i] * Elem<T>::load(row, g * D + i);
            tot += dq * rn[g];
        }
        best = fmaxf(best, tot * inv_hq);
    }
    cout[b * N + n] = best;
}

template <typename T, int D>
hipError_t launch_scan_generic(const RouteArgs& a, const float* U, float* c, hipStream_t st) {
    const int64_t total = a.B * a.N;
    return launch_timed(route_scan_generic<T, D>, dim3(unsigned(ceil_div(total, 256))), dim3(256), st,
                        a.prof_start, a.prof_stop, static_cast<const T*>(a.Krbar), a.N, a.Hkv, U, a.B, a.Tq,
                        1.f / float(a.Hq), c);
}

bool qr_aligned16(const RouteArgs& a) { return (reinterpret_cast<uintptr_t>(a.Qr) & 15u) == 0; }

template <int LPR, int NQ>
hipError_t launch_scan_fast(const RouteArgs& a, const float* U, float* c, hipStream_t st) {
    const int64_t groups = ceil_div(a.N, 64);
    int64_t blocks = ceil_div(groups, 4);
    const int64_t cap = int64_t(a.num_cus) * 4;   // 16 waves per CU, grid-strided over 64-row groups
    if (blocks > cap) blocks = cap;
    const u32x4* qr = static_cast<const u32x4*>(a.Qr);
    if (qr_aligned16(a))
        return launch_timed(route_scan_bf16_d128<LPR, NQ, true>, dim3(unsigned(blocks)), dim3(256), st,
                            a.prof_start, a.prof_stop, static_cast<const u32x4*>(a.Krbar), a.N, U, qr, a.Hq,
                            int(a.B), a.Tq, 1.f / float(a.Hq), c);
    return launch_timed(route_scan_bf16_d128<LPR, NQ, false>, dim3(unsigned(blocks)), dim3(256), st,
                        a.prof_start, a.prof_stop, static_cast<const u32x4*>(a.Krbar), a.N, U, qr, a.Hq,
                        int(a.B), a.Tq, 1.f / float(a.Hq), c);
}

template <int LPR>
hipError_t dispatch_nq(const RouteArgs& a, const float* U, float* c, hipStream_t st) {
    switch (a.B * a.Tq) {
        case 1: return launch_scan_fast<LPR, 1>(a, U, c, st);
        case 2: return launch_scan_fast<LPR, 2>(a, U, c, st);
        case 3: return launch_scan_fast<LPR, 3>(a, U, c, st);
        default: return launch_scan_fast<LPR, 4>(a, U, c, st);
    }
}


}  // namespace

bool route_generic_supported(int Hkv) { return Hkv <= kMaxHkvGeneric; }

hipError_t launch_route_prep(const RouteArgs& a, float* U, hipStream_t st) {
    const unsigned grid = unsigned(a.B * a.Tq * a.Hkv);
    if (a.dt == MSA_BF16 && a.D == 128 && (reinterpret_cast<uintptr_t>(a.Qr) & 15u) == 0) {
        const int64_t items = a.B * a.Tq * a.Hkv;
        int64_t blocks = ceil_div(items, int64_t(4));
        const int64_t cap = int64_t(a.num_cus) * 8;
        if (blocks > cap) blocks = cap;
        hipLaunchKernelGGL(route_prep_bf16_d128, dim3(unsigned(blocks < 1 ? 1 : blocks)), dim3(256), 0, st,
                           static_cast<const u32x4*>(a.Qr), items, a.Hq, a.Hkv, U);
        return hipGetLastError();
    }
    if (a.dt == MSA_BF16) {
        if (a.D == 128)
            hipLaunchKernelGGL((route_prep_kernel<bf16_t, 128>), dim3(grid), dim3(64), 0, st,
                               static_cast<const bf16_t*>(a.Qr), a.Hq, a.Hkv, U);
        else
            hipLaunchKernelGGL((route_prep_kernel<bf16_t, 64>), dim3(grid), dim3(64), 0, st,
                               static_cast<const bf16_t*>(a.Qr), a.Hq, a.Hkv, U);
    } else {
        if (a.D == 128)
            hipLaunchKernelGGL((route_prep_kernel<float, 128>), dim3(grid), dim3(64), 0, st,
                               static_cast<const float*>(a.Qr), a.Hq, a.Hkv, U);
        else
            hipLaunchKernelGGL((route_prep_kernel<float, 64>), dim3(grid), dim3(64), 0, st,
                               static_cast<const float*>(a.Qr), a.Hq, a.Hkv, U);
    }
    return hipGetLastError();
}

bool route_scan_fast_applicable(const RouteArgs& a) {
    return a.dt == MSA_BF16 && a.D == 128 && a.B * a.Tq <= 4 &&
           (a.Hkv == 4 || a.Hkv == 8 || a.Hkv == 16);
}

bool route_scan_fast_preps_itself(const RouteArgs& a) { return route_scan_fast_applicable(a) && qr_aligned16(a); }

hipError_t launch_route_scan_fast(const RouteArgs& a, const float* U, float* c, hipStream_t st) {
    if (a.Hkv == 4) return dispatch_nq<1>(a, U, c, st);
    if (a.Hkv == 8) return dispatch_nq<2>(a, U, c, st);
    return dispatch_nq<4>(a, U, c, st);
}

hipError_t launch_route_scan_generic(const RouteArgs& a, const float* U, float* c,
                                     hipStream_t st) {
    if (a.dt == MSA_BF16)
        return (a.D == 128) ? launch_scan_generic<bf16_t, 128>(a, U, c, st)
                            : launch_scan_generic<bf16_t, 64>(a, U, c, st);
    return (a.D == 128) ? launch_scan_generic<float, 128>(a, U, c, st)
                        : launch_scan_generic<float, 64>(a, U, c, st);
}

}  // namespace msa
