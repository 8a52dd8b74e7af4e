// Stage 2a on the matrix cores: routing scores as a dense contraction, for
// batched decode (B*Tq > 4, Tq = 1) and multi-token query prefill (Tq a
// multiple of 128).
//
// Source: news.neo-ai.one MSA article, 全体設計 › アーキテクチャ (Fig. 2):
// cosine similarity of Qr with K̄r, averaged over heads, maximised over
// tokens.  With U[q][g] = sum_{h in g} q_h / max(|q_h|, eps) (route_prep), the
// score of query token q and chunk n is
//     s[q][n] = (1/Hq) sum_g rn[n][g] * (U[q][g] . K̄r[n][g]),
//     rn[n][g] = 1 / max(|K̄r[n][g]|, eps),
// i.e. a [Q x (Hkv*128)] x [(Hkv*128) x N] product whose 128-wide slices are
// scaled per (chunk, head group) before they are summed.
//
// route_mfma_kernel<BM, BN>: a workgroup (4 waves) owns a BM x BN tile of
// (query tokens) x (chunks).  For each head group g it stages the bf16 U and
// K̄r slices (128 wide) in LDS with 16-byte loads, computes the chunks' rn from
// the same loads (16-lane DPP sums of squares), runs 8 k-steps of
// v_mfma_f32_32x32x16_bf16 into a per-group accumulator, and adds rn times
// that accumulator to the running total.  K̄r enters the MFMA exactly; U is
// rounded once to bf16 (relative error <= 2^-9 per element), which moves a
// score by at most (1/Hq) sum_g 2^-9 |U_g| <= 2^-9, since |U_g| <= G.
// Epilogue: Tq = 1 -> each row is its own query, scores are written; Tq a
// multiple of BM -> the tile's column maxima over its BM tokens are written
// to a partial array and route_mfma_tokmax takes the max over a query's tiles.
#include "route_mfma.hpp"

namespace msa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kStride = 128 + 8;   // LDS row stride in bf16 (16-byte pad: 4-bank skew per row)
constexpr float kEps = 1e-8f;

__global__ __launch_bounds__(256) void u_to_bf16_kernel(const float* __restrict__ U, int64_t n_real,
                                                        int64_t n_pad, uint16_t* __restrict__ Ub) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n_pad) return;
    Ub[i] = (i < n_real) ? f32_to_bf16(U[i]) : uint16_t(0);
}

// Tile order.  Workgroups are dealt to the 8 XCDs round-robin by linear id, and
// each XCD has its own L2.  Consecutive workgroups of one XCD take the tiles of
// one super-tile of SQ query tiles x SC chunk tiles, so the tiles in flight on
// an XCD share their U and K̄r slices through its L2 (at 128 x 128 tiles and
// SQ = SC = 8: 2 MB of U + 2 MB of K̄r), and K̄r is streamed from HBM once per
// super-tile row instead of once per query tile.
constexpr int kXcds = 8;

struct TileOrder {
    int64_t tq, tn;          // query tiles, chunk tiles
    int sq, sc;              // super-tile extent (query tiles, chunk tiles)
    int64_t n_sq;            // super-tiles along the queries
    int64_t blocks;          // grid size (a multiple of kXcds * sq * sc)
};

__host__ __device__ inline TileOrder tile_order(int64_t tq, int64_t tn) {
    TileOrder o;
    o.tq = tq; o.tn = tn;
    o.sq = tq < 8 ? int(tq) : 8;
    o.sc = 8;
    o.n_sq = (tq + o.sq - 1) / o.sq;
    const int64_t n_super = o.n_sq * ((tn + o.sc - 1) / o.sc);
    o.blocks = ((n_super + kXcds - 1) / kXcds) * kXcds * o.sq * o.sc;
    return o;
}

// rn[n][g] = 1 / max(|K̄r[n][g]|, eps), for the prefill path, where every chunk
// tile is used by many query tiles: 16 lanes per 128-wide slice, the same
// per-lane sums and DPP reduction as the inline form in route_mfma_kernel.
__global__ __launch_bounds__(256) void route_rnorm_kernel(const uint16_t* __restrict__ Kr, int64_t n_slices,
                                                          float* __restrict__ rn) {
    const int64_t slice = (int64_t(blockIdx.x) * 256 + threadIdx.x) / 16;
    const int c = threadIdx.x % 16;
    const int64_t sl = slice < n_slices ? slice : n_slices - 1;
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Kr + sl * 128 + c * 8));
    float s = 0.f, f;
    f = bf16_lo(v.x); s += f * f; f = bf16_hi(v.x); s += f * f;
    f = bf16_lo(v.y); s += f * f; f = bf16_hi(v.y); s += f * f;
    f = bf16_lo(v.z); s += f * f; f = bf16_hi(v.z); s += f * f;
    f = bf16_lo(v.w); s += f * f; f = bf16_hi(v.w); s += f * f;
    s = group_sum<16>(s);
    if (c == 0 && slice < n_slices) rn[slice] = __builtin_amdgcn_rsqf(fmaxf(s, kEps * kEps));
}

template <int BM, int BN, bool PRE_RN>
__global__ __launch_bounds__(256, 2) void route_mfma_kernel(
    const uint16_t* __restrict__ Ub, int64_t Q, const uint16_t* __restrict__ Kr, int64_t N, int hkv,
    int Tq, float inv_hq, float* __restrict__ cout, float* __restrict__ partial, TileOrder ord,
    const float* __restrict__ rn_pre) {
    constexpr int WM = (BM >= 64) ? 2 : 1;        // waves along queries
    constexpr int WN = 4 / WM;                    // waves along chunks
    constexpr int TM = BM / WM, TN = BN / WN;     // wave tile
    constexpr int MI = TM / 32, NI = TN / 32;     // 32x32 MFMA tiles per wave
    constexpr int RU = BM * 16 / 256, RK = BN * 16 / 256;   // 16-byte pieces per thread
    __shared__ __attribute__((aligned(16))) uint16_t sU[BM * kStride];
    __shared__ __attribute__((aligned(16))) uint16_t sK[BN * kStride];
    __shared__ float sRn[BN];
    __shared__ float sMax[WM][BN];

    // ---- which tile (see TileOrder)
    const int64_t lin = blockIdx.x;
    const int xcd = int(lin % kXcds);
    const int64_t loc = lin / kXcds;
    const int per = ord.sq * ord.sc;
    const int64_t sup = (loc / per) * kXcds + xcd;
    const int w = int(loc % per);
    const int64_t qt = (sup % ord.n_sq) * ord.sq + w % ord.sq;
    const int64_t ct = (sup / ord.n_sq) * ord.sc + w / ord.sq;
    if (qt >= ord.tq || ct >= ord.tn) return;     // whole workgroup: padding of the grid

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int wm = wave / WN, wn = wave % WN;
    const int64_t n0 = ct * BN;
    const int64_t q0 = qt * BM;
    const int64_t row_elems = int64_t(hkv) * 128;
    const int c = tid % 16;                       // 16-byte column of a 128-wide slice

    f32x16 tot[MI][NI], acc[MI][NI];
    const f32x16 zero = {};
#pragma unroll
    for (int a = 0; a < MI; ++a)
#pragma unroll
        for (int b = 0; b < NI; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) tot[a][b][i] = 0.f;

    // ---- register prefetch of one head group's U and K̄r slices
    u32x4 ru[RU], rk[RK];
    auto fetch = [&](int g) {
#pragma unroll
        for (int j = 0; j < RU; ++j) {
            const int r = tid / 16 + 16 * j;
            ru[j] = *reinterpret_cast<const u32x4*>(Ub + (q0 + r) * row_elems + g * 128 + c * 8);
        }
#pragma unroll
        for (int j = 0; j < RK; ++j) {
            int64_t n = n0 + tid / 16 + 16 * j;
            n = n < N ? n : N - 1;                   // tail rows: computed, never stored
            rk[j] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(Kr + n * row_elems + g * 128 + c * 8));
        }
    };
    fetch(0);

    for (int g = 0; g < hkv; ++g) {
        // ---- slices of group g to LDS; norms of the K̄r slices
#pragma unroll
        for (int j = 0; j < RU; ++j)
            *reinterpret_cast<u32x4*>(sU + (tid / 16 + 16 * j) * kStride + c * 8) = ru[j];
#pragma unroll
        for (int j = 0; j < RK; ++j) {
            const int r = tid / 16 + 16 * j;
            const u32x4 v = rk[j];
            *reinterpret_cast<u32x4*>(sK + r * kStride + c * 8) = v;
            if constexpr (PRE_RN) continue;
            float s = 0.f, f;
            f = bf16_lo(v.x); s += f * f; f = bf16_hi(v.x); s += f * f;
            f = bf16_lo(v.y); s += f * f; f = bf16_hi(v.y); s += f * f;
            f = bf16_lo(v.z); s += f * f; f = bf16_hi(v.z); s += f * f;
            f = bf16_lo(v.w); s += f * f; f = bf16_hi(v.w); s += f * f;
            s = group_sum<16>(s);
            if (c == 0) sRn[r] = __builtin_amdgcn_rsqf(fmaxf(s, kEps * kEps));
        }
        __syncthreads();
        if (g + 1 < hkv) fetch(g + 1);               // in flight during this group's MFMAs

        // ---- 128-deep contraction of this group on the matrix cores
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int col = ks * 16 + (lane / 32) * 8;
            bf16x8 af[MI], bfr[NI];
#pragma unroll
            for (int a = 0; a < MI; ++a)
                af[a] = *reinterpret_cast<const bf16x8*>(sU + (wm * TM + a * 32 + lane % 32) * kStride + col);
#pragma unroll
            for (int b = 0; b < NI; ++b)
                bfr[b] = *reinterpret_cast<const bf16x8*>(sK + (wn * TN + b * 32 + lane % 32) * kStride + col);
#pragma unroll
            for (int a = 0; a < MI; ++a)
#pragma unroll
                for (int b = 0; b < NI; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], ks == 0 ? zero : acc[a][b],
                                                                        0, 0, 0);
        }
        // ---- scale by 1/|K̄r[n][g]| (one chunk column per lane) and accumulate
#pragma unroll
        for (int b = 0; b < NI; ++b) {
            float rn;
            if constexpr (PRE_RN) {
                int64_t n = n0 + wn * TN + b * 32 + lane % 32;
                n = n < N ? n : N - 1;
                rn = rn_pre[n * hkv + g];
            } else {
                rn = sRn[wn * TN + b * 32 + lane % 32];
            }
#pragma unroll
            for (int a = 0; a < MI; ++a)
#pragma unroll
                for (int i = 0; i < 16; ++i) tot[a][b][i] += rn * acc[a][b][i];
        }
        __syncthreads();
    }

    // ---- epilogue
    if (Tq == 1) {
#pragma unroll
        for (int a = 0; a < MI; ++a)
#pragma unroll
            for (int b = 0; b < NI; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int64_t q = q0 + wm * TM + a * 32 + (i / 4) * 8 + (lane / 32) * 4 + (i % 4);
                    const int64_t n = n0 + wn * TN + b * 32 + lane % 32;
                    if (q < Q && n < N) cout[q * N + n] = tot[a][b][i] * inv_hq;
                }
        return;
    }
#pragma unroll
    for (int b = 0; b < NI; ++b) {
        float m = -INFINITY;
#pragma unroll
        for (int a = 0; a < MI; ++a)
#pragma unroll
            for (int i = 0; i < 16; ++i) m = fmaxf(m, tot[a][b][i]);
        m = fmaxf(m, __shfl_xor(m, 32));
        if (lane < 32) sMax[wm][wn * TN + b * 32 + lane] = m;
    }
    __syncthreads();
    for (int t = tid; t < BN; t += 256) {
        float m = sMax[0][t];
#pragma unroll
        for (int w = 1; w < WM; ++w) m = fmaxf(m, sMax[w][t]);
        const int64_t n = n0 + t;
        if (n < N) partial[qt * N + n] = m * inv_hq;
    }
}

// c[b][n] = max over the query's tiles of partial[tile][n]
__global__ __launch_bounds__(256) void route_mfma_tokmax(const float* __restrict__ partial, int64_t N,
                                                         int tiles_per_query, int64_t B, float* __restrict__ cout) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= B * N) return;
    const int64_t b = i / N, n = i % N;
    float m = -INFINITY;
    for (int t = 0; t < tiles_per_query; ++t) m = fmaxf(m, partial[(b * tiles_per_query + t) * N + n]);
    cout[i] = m;
}

struct Plan {
    int bm, bn;
    int64_t q_pad, q_tiles;
    size_t ub_bytes, partial_bytes, rn_bytes;
};

Plan plan_for(int64_t B, int Tq, int Hkv, int64_t N) {
    Plan p;
    const int64_t Q = B * Tq;
    p.bm = (Tq == 1 && Q <= 32) ? 32 : 128;
    p.bn = 128;
    p.q_pad = ceil_div(Q, p.bm) * p.bm;
    p.q_tiles = p.q_pad / p.bm;
    p.ub_bytes = align256(size_t(p.q_pad) * Hkv * 128 * 2);
    p.partial_bytes = (Tq == 1) ? 0 : align256(size_t(p.q_tiles) * N * 4);
    p.rn_bytes = (p.q_tiles > 1) ? align256(size_t(N) * Hkv * 4) : 0;   // norms computed once, shared by the query tiles
    return p;
}

}  // namespace

bool route_mfma_applicable(msa_dtype dt, int64_t B, int Tq, int Hkv, int D) {
    if (dt != MSA_BF16 || D != 128 || Hkv < 1) return false;
    if (B * Tq <= 4) return false;                 // the streaming scan handles decode
    return Tq == 1 || Tq % 128 == 0;
}

size_t route_mfma_workspace(msa_dtype dt, int64_t B, int Tq, int Hq, int Hkv, int D, int64_t N, int) {
    (void)Hq;
    if (!route_mfma_applicable(dt, B, Tq, Hkv, D)) return 0;
    const Plan p = plan_for(B, Tq, Hkv, N);
    return p.ub_bytes + p.partial_bytes + p.rn_bytes;
}

hipError_t launch_route_mfma(const RouteArgs& a, const float* U, float* c, void* ws, hipStream_t st) {
    const Plan p = plan_for(a.B, a.Tq, a.Hkv, a.N);
    const int64_t Q = a.B * a.Tq;
    uint16_t* Ub = static_cast<uint16_t*>(ws);
    float* partial = reinterpret_cast<float*>(static_cast<char*>(ws) + p.ub_bytes);
    float* rn = reinterpret_cast<float*>(static_cast<char*>(ws) + p.ub_bytes + p.partial_bytes);
    const int64_t n_real = Q * a.Hkv * 128, n_pad = p.q_pad * a.Hkv * 128;
    hipLaunchKernelGGL(u_to_bf16_kernel, dim3(unsigned(ceil_div(n_pad, 256))), dim3(256), 0, st, U, n_real,
                       n_pad, Ub);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const TileOrder ord = tile_order(p.q_tiles, ceil_div(a.N, p.bn));
    const dim3 grid(unsigned(ord.blocks));
    const float inv_hq = 1.f / float(a.Hq);
    const uint16_t* Kr = static_cast<const uint16_t*>(a.Krbar);
    if (p.rn_bytes) {
        const int64_t n_slices = a.N * a.Hkv;
        hipLaunchKernelGGL(route_rnorm_kernel, dim3(unsigned(ceil_div(n_slices * 16, 256))), dim3(256), 0, st, Kr,
                           n_slices, rn);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (p.bm == 32) {
        if (p.rn_bytes)
            hipLaunchKernelGGL((route_mfma_kernel<32, 128, true>), grid, dim3(256), 0, st, Ub, Q, Kr, a.N, a.Hkv,
                               a.Tq, inv_hq, c, partial, ord, rn);
        else
            hipLaunchKernelGGL((route_mfma_kernel<32, 128, false>), grid, dim3(256), 0, st, Ub, Q, Kr, a.N, a.Hkv,
                               a.Tq, inv_hq, c, partial, ord, rn);
    } else {
        if (p.rn_bytes)
            hipLaunchKernelGGL((route_mfma_kernel<128, 128, true>), grid, dim3(256), 0, st, Ub, Q, Kr, a.N, a.Hkv,
                               a.Tq, inv_hq, c, partial, ord, rn);
        else
            hipLaunchKernelGGL((route_mfma_kernel<128, 128, false>), grid, dim3(256), 0, st, Ub, Q, Kr, a.N, a.Hkv,
                               a.Tq, inv_hq, c, partial, ord, rn);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (a.Tq > 1) {
        hipLaunchKernelGGL(route_mfma_tokmax, dim3(unsigned(ceil_div(a.B * a.N, 256))), dim3(256), 0, st, partial,
                           a.N, int(a.Tq / p.bm), a.B, c);
        err = hipGetLastError();
    }
    return err;
}

}  // namespace msa
