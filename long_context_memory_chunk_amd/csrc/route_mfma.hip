// Stage 2a on the matrix cores: routing scores as a dense contraction, for
// batched decode (B*Tq > 4) and multi-token query prefill of any length.  Two
// kernels: route_mfma_kernel (below) for decode batches and short query
// blocks, and the one-GEMM path (route_gemm_kernel, further down) for long
// queries (Tq a multiple of 256, or at least 1,024 tokens).
//
// A multi-token query is padded to a whole number of row tiles: query b's
// token t sits at row b * Tq_pad + t, rows t >= Tq hold zeros and are left
// out of the token max (a tile never holds two queries, and the last tile of
// a query holds at least one real token).
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
// Epilogue: Tq = 1 -> each row is its own query, scores are written; else ->
// the tile's column maxima over its real tokens are written to a partial
// array and route_mfma_tokmax takes the max over a query's tiles.
#include <type_traits>

#include "lds_dma.hpp"
#include "route_mfma.hpp"

namespace msa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kStride = 128 + 8;   // LDS row stride in bf16 (16-byte pad: 4-bank skew per row)
constexpr float kEps = 1e-8f;

// U rows in the padded layout: padded row p is query p / Tq_pad's token
// p % Tq_pad, real when that token is < Tq (and the query < B).
__host__ __device__ inline int64_t u_src_row(int64_t p, int64_t B, int Tq, int Tq_pad) {
    const int64_t b = p / Tq_pad;
    const int t = int(p % Tq_pad);
    return (b < B && t < Tq) ? b * Tq + t : -1;
}

__global__ __launch_bounds__(256) void u_to_bf16_kernel(const float* __restrict__ U, int64_t B, int Tq, int Tq_pad,
                                                        int row_elems, int64_t n_pad, uint16_t* __restrict__ Ub) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n_pad) return;
    const int64_t src = u_src_row(i / row_elems, B, Tq, Tq_pad);
    Ub[i] = (src >= 0) ? f32_to_bf16(U[src * row_elems + i % row_elems]) : uint16_t(0);
}

// route_prep and the bf16 rounding in one launch, for route_mfma_kernel:
// padded row p, group g of Ub holds U[q][g] = sum_{h in g} q_h / max(|q_h|,
// eps) of query token q = u_src_row(p), rounded to bf16 (zeros for a padding
// row).  bf16 rows of 128: lane l loads the 16-byte slot l % 16 of head l / 16
// of a batch of four heads (one 1 KB wave load per batch), each head's norm is
// a 16-lane sum, the four partial rows meet by two shuffles, and lanes 0..15
// store the group's 128 values.  The head sum is taken in the order of
// route_prep's 16-byte form, so Ub holds the bits u_to_bf16 would give.
__global__ __launch_bounds__(256) void route_prep_ub_kernel(const u32x4* __restrict__ Qr, int64_t B, int Tq,
                                                            int Tq_pad, int64_t n_items, int Hq, int hkv,
                                                            u32x4* __restrict__ Ub) {
    const int G = Hq / hkv;
    const int lane = threadIdx.x % kWave, sub = lane / 16, c = lane % 16;
    for (int64_t it = int64_t(blockIdx.x) * 4 + threadIdx.x / kWave; it < n_items; it += int64_t(gridDim.x) * 4) {
        const int64_t prow = it / hkv;
        const int g = int(it % hkv);
        const int64_t q = u_src_row(prow, B, Tq, Tq_pad);
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        if (q >= 0) {
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
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[e] += __shfl_xor(acc[e], 16);
            acc[e] += __shfl_xor(acc[e], 32);
        }
        if (sub == 0)
            Ub[(prow * hkv + g) * 16 + c] = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                                  pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
    }
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

__host__ __device__ inline TileOrder tile_order(int64_t tq, int64_t tn, int sq_max = 8, int sc = 8) {
    TileOrder o;
    o.tq = tq; o.tn = tn;
    o.sq = tq < sq_max ? int(tq) : sq_max;
    o.sc = sc;
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
    int Tq, int Tq_pad, float inv_hq, float* __restrict__ cout, float* __restrict__ partial, TileOrder ord,
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
    float rnv = 0.f;                                  // precomputed norm of chunk n0 + tid (tid < BN)
    auto fetch = [&](int g) {
        if constexpr (PRE_RN) {
            if (tid < BN) {
                int64_t n = n0 + tid;
                n = n < N ? n : N - 1;
                rnv = rn_pre[n * hkv + g];
            }
        }
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
        if constexpr (PRE_RN) {
            if (tid < BN) sRn[tid] = rnv;
        }
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
            const float rn = sRn[wn * TN + b * 32 + lane % 32];
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
    // rows of this tile that are real tokens of its query (the padding of a
    // query's last tile is left out of the max)
    const int64_t t_in = q0 % Tq_pad;
    const int real = (Tq - t_in < BM) ? int(Tq - t_in) : BM;
#pragma unroll
    for (int b = 0; b < NI; ++b) {
        float m = -INFINITY;
#pragma unroll
        for (int a = 0; a < MI; ++a)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = wm * TM + a * 32 + (i / 4) * 8 + (lane / 32) * 4 + (i % 4);
                m = (r < real) ? fmaxf(m, tot[a][b][i]) : m;
            }
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

// ---------------------------------------------------------------- prefill: one GEMM
//
// For a long prefill query (padded to a multiple of 256) the scores are computed as one
// bf16 GEMM over the full Hkv*128-wide contraction,
//     s[q][n] = (1/Hq) U[q] . K̂[n],   K̂[n][g] = K̄r[n][g] / max(|K̄r[n][g]|, eps),
// with K̂ rounded once to bf16 by route_khat_pack (a second rounding next to
// U's; the score moves by at most 2^-9 + 2^-9 = 2^-8).  Both operands are first
// written in a packed tile layout: for a 256-row tile and a 32-wide stage of the
// contraction, one 16 KB block in which the 16-byte unit u of row r sits at
// unit r*4 + (u ^ swz(r)).  route_gemm_kernel then copies each block into LDS
// with direct global->LDS loads (lane i of a wave writes LDS base + 16 i, so a
// contiguous copy reproduces the layout) into a ring of four stages, three
// copies in flight behind the stage in use, and the XOR swizzle makes the rows
// of a matrix-core operand read hit distinct LDS banks.  A workgroup (4 waves,
// 2 x 2) owns 256 queries x 256 chunks; a wave owns 128 x 128, 16 accumulator
// tiles of v_mfma_f32_32x32x16_bf16.  Each stage is two k-steps of 16, 32
// products per wave; the next stage's operands are read into a second register
// set, and the copies of the stage three ahead issued, a few at a time between
// groups of products (see the pipeline below).  The epilogue writes the tile's
// column maxima over its 256 tokens.

constexpr int GB = 256;          // GEMM tile rows (queries and chunks)
constexpr int GK = 32;           // contraction width of one stage
constexpr int GU = GK / 8;       // 16-byte units per row of a stage
constexpr int kUnitsPerStage = GB * GU;       // 16-byte units of one operand stage (1024 = 16 KB)
constexpr int kStages = 4;       // stages in LDS: three copies in flight behind the one in use

// Row r's unit u sits at unit r*GU + (u ^ swz(r)), swz(r) = (r ^ (r >> 2)) & 3,
// so the rows of one operand read fall in distinct LDS banks.  (Measured with
// the SQ_LDS_BANK_CONFLICT counter on the 8K prefill: 0 conflict cycles, where
// ((r >> 1) ^ (r >> 3)) & 3 gave 160M and a 9% slower kernel.)
__host__ __device__ inline int swz(int r) { return (r ^ (r >> 2)) & 3; }

// U (fp32 [B*Tq][K]) -> packed bf16 tiles in the padded row layout; padding
// rows are zero.  One thread per unit.
__global__ __launch_bounds__(256) void route_u_pack(const float* __restrict__ U, int64_t B, int Tq, int Tq_pad,
                                                    int64_t q_pad, int K, u32x4* __restrict__ Up) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;        // unit index in row-major order
    const int units_per_row = K / 8;
    if (i >= q_pad * units_per_row) return;
    const int64_t q = i / units_per_row;
    const int ku = int(i % units_per_row);                             // unit along the contraction
    u32x4 w = {0u, 0u, 0u, 0u};
    const int64_t sq = u_src_row(q, B, Tq, Tq_pad);
    if (sq >= 0) {
        const float* src = U + sq * K + ku * 8;
        w = u32x4{pack_bf16x2(src[0], src[1]), pack_bf16x2(src[2], src[3]), pack_bf16x2(src[4], src[5]),
                  pack_bf16x2(src[6], src[7])};
    }
    const int64_t tile = q / GB;
    const int r = int(q % GB), st = ku / GU, u = ku % GU;
    const int S = K / GK;
    Up[(tile * S + st) * kUnitsPerStage + r * GU + (u ^ swz(r))] = w;
}

// K̄r (bf16 [N][Hkv][128]) -> normalised, packed bf16 tiles of K̂; rows >= N are
// zero.  16 lanes per 128-wide slice: the slice norm is reduced across them.
__global__ __launch_bounds__(256) void route_khat_pack(const uint16_t* __restrict__ Kr, int64_t N, int64_t n_pad,
                                                       int hkv, u32x4* __restrict__ Kp) {
    const int64_t slice = (int64_t(blockIdx.x) * 256 + threadIdx.x) / 16;  // (n, g) in [0, n_pad * hkv)
    const int c = threadIdx.x % 16;
    if (slice >= n_pad * hkv) return;                                       // whole 16-lane groups
    const int64_t n = slice / hkv;
    const int g = int(slice % hkv);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n < N) v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Kr + slice * 128 + c * 8));
    float x[8];
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
    ss = group_sum<16>(ss);
    const float rn = __builtin_amdgcn_rsqf(fmaxf(ss, kEps * kEps));
    const u32x4 w = {pack_bf16x2(x[0] * rn, x[1] * rn), pack_bf16x2(x[2] * rn, x[3] * rn),
                     pack_bf16x2(x[4] * rn, x[5] * rn), pack_bf16x2(x[6] * rn, x[7] * rn)};
    const int ku = g * 16 + c;                                               // unit along the contraction
    const int64_t tile = n / GB;
    const int r = int(n % GB), st = ku / GU, u = ku % GU;
    const int S = hkv * 128 / GK;
    Kp[(tile * S + st) * kUnitsPerStage + r * GU + (u ^ swz(r))] = w;
}

__global__ __launch_bounds__(256, 1) void route_gemm_kernel(const u32x4* __restrict__ Up, const u32x4* __restrict__ Kp,
                                                            int64_t N, int S, int Tq, int Tq_pad, float inv_hq,
                                                            float* __restrict__ partial, TileOrder ord) {
    __shared__ __attribute__((aligned(16))) u32x4 sA[kStages * kUnitsPerStage];
    __shared__ __attribute__((aligned(16))) u32x4 sB[kStages * kUnitsPerStage];
    __shared__ float sMax[2][GB];

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
    const int wm = wave / 2, wn = wave % 2;
    const u32x4* Ag = Up + qt * int64_t(S) * kUnitsPerStage;
    const u32x4* Bg = Kp + ct * int64_t(S) * kUnitsPerStage;
    const uint32_t ldsA = lds_addr(sA), ldsB = lds_addr(sB);

    // one stage = 2 x 16 KB; a wave copies 4 + 4 contiguous 1 KB pieces (8 copies),
    // addressed as scalar bases plus the lane's 16-byte offset
    constexpr int kCopies = 8;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t voff = uint32_t(lane) * 16u;
    auto dma = [&](int st) {
        const u32x4* a = Ag + int64_t(st) * kUnitsPerStage;
        const u32x4* b = Bg + int64_t(st) * kUnitsPerStage;
        const uint32_t buf = uint32_t(st % kStages) * kUnitsPerStage;
#pragma unroll
        for (int i = 0; i < kCopies / 2; ++i) {
            const int piece = (i * 4 + wave_u) * kWave;
            lds_copy16_s(a + piece, voff, ldsA + (buf + piece) * 16);
            lds_copy16_s(b + piece, voff, ldsB + (buf + piece) * 16);
        }
    };

    // operand addresses (units) inside a stage: row r, unit (2 ks + lane/32) ^ swz(r)
    int offA[4], offB[4], sw[8];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int ra = wm * 128 + a * 32 + lane % 32;
        const int rb = wn * 128 + a * 32 + lane % 32;
        offA[a] = ra * GU;
        offB[a] = rb * GU;
        sw[a] = swz(ra) ^ (lane / 32);
        sw[4 + a] = swz(rb) ^ (lane / 32);
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

    // Software pipeline, one stage (two 16-deep k-steps) of operands ahead in
    // registers.  Stage st:
    //   wait for stage st + 1's copies (only stage st + 2's may remain in
    //   flight), barrier;
    //   copy stage st + 3 into the buffer of stage st - 1, whose operands every
    //   wave read into registers during stage st - 2 and consumed in stage
    //   st - 1, before this barrier;
    //   read stage st + 1's operands into the other register set while the
    //   matrix cores run stage st's 32 products, so a read has a whole stage
    //   to complete.
    // Operand sets P and Q alternate between stages: [k-step][32-row tile].
    bf16x8 pa[2][4], pb[2][4], qa[2][4], qb[2][4];
    constexpr int kReadFrom[9] = {0, 3, 6, 9, 12, 14, 16, 16, 16};
    // copy j (0..7) of stage st: piece j / 2 of operand A (j even) or B (j odd)
    auto dma_one = [&](int st, int j) {
        const int piece = ((j >> 1) * 4 + wave_u) * kWave;
        const uint32_t buf = uint32_t(st % kStages) * kUnitsPerStage;
        if (j & 1) lds_copy16_s(Bg + int64_t(st) * kUnitsPerStage + piece, voff, ldsB + (buf + piece) * 16);
        else lds_copy16_s(Ag + int64_t(st) * kUnitsPerStage + piece, voff, ldsA + (buf + piece) * 16);
    };
// Read r (0..15) of stage st's operands: k-step r / 8, tile (r / 2) % 4, A or B.
#define MSA_GEMM_READ_ONE(st_, r_, RA, RB)                                                 \
    {                                                                                      \
        const int ks_ = (r_) / 8, t_ = ((r_) / 2) % 4;                                     \
        if ((r_) & 1)                                                                      \
            RB[ks_][t_] = __builtin_bit_cast(bf16x8, sB[((st_) % kStages) * kUnitsPerStage + offB[t_] + ((2 * ks_) ^ sw[4 + t_])]); \
        else                                                                               \
            RA[ks_][t_] = __builtin_bit_cast(bf16x8, sA[((st_) % kStages) * kUnitsPerStage + offA[t_] + ((2 * ks_) ^ sw[t_])]);     \
    }
// One stage: wait until at most WAITN copies are in flight (stage s + 1
// resident), barrier; then eight groups of four of stage s's products from
// (CA, CB), each followed by one copy of stage s + 3 (DO_DMA) and some of the
// 16 operand reads of stage s + 1 into (NA, NB) (DO_READ: 3, 3, 3, 3, 2, 2 in
// the first six groups, so the last reads have two groups of products to land
// before the next barrier waits for them).  Spreading the copies and
// reads over the stage keeps every wave's in-order issue moving: issued all at
// once after the barrier, the four waves' 32 copies queue at the CU's address
// unit and hold back the products behind them.  The scheduling barriers keep
// that order.
#define MSA_GEMM_STEP(st_, CA, CB, NA, NB, WAITN, DO_DMA, DO_READ)                          \
    {                                                                                      \
        const int s_ = (st_);                                                              \
        if (DO_READ) {                                                                     \
            MSA_WAIT_VMCNT(WAITN);                                                         \
            __syncthreads();                                                               \
        }                                                                                  \
        _Pragma("unroll") for (int g = 0; g < 8; ++g) {                                    \
            _Pragma("unroll") for (int m = 4 * g; m < 4 * g + 4; ++m)                      \
                acc[(m / 4) % 4][m % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(          \
                    CA[m / 16][(m / 4) % 4], CB[m / 16][m % 4], acc[(m / 4) % 4][m % 4], 0, 0, 0); \
            if (DO_DMA) dma_one(s_ + kStages - 1, g);                                      \
            if (DO_READ)                                                                   \
                _Pragma("unroll") for (int r = kReadFrom[g]; r < kReadFrom[g + 1]; ++r)    \
                    MSA_GEMM_READ_ONE(s_ + 1, r, NA, NB)                                   \
            __builtin_amdgcn_sched_barrier(0);                                             \
        }                                                                                  \
    }

    // S = Hkv * 4 stages, a multiple of 4: stages 0 .. S - 5 in pairs with every
    // step whole, then the last four peeled (the copies run out three stages
    // before the products do).
    for (int st = 0; st < kStages - 1; ++st) dma(st);
    MSA_WAIT_VMCNT(2 * kCopies);
    __syncthreads();
    _Pragma("unroll") for (int r = 0; r < 16; ++r) MSA_GEMM_READ_ONE(0, r, pa, pb)
    for (int st = 0; st + 4 < S; st += 2) {
        MSA_GEMM_STEP(st, pa, pb, qa, qb, kCopies, true, true)
        MSA_GEMM_STEP(st + 1, qa, qb, pa, pb, kCopies, true, true)
    }
    MSA_GEMM_STEP(S - 4, pa, pb, qa, qb, kCopies, true, true)
    MSA_GEMM_STEP(S - 3, qa, qb, pa, pb, kCopies, false, true)
    MSA_GEMM_STEP(S - 2, pa, pb, qa, qb, 0, false, true)
    MSA_GEMM_STEP(S - 1, qa, qb, pa, pb, 0, false, false)
#undef MSA_GEMM_STEP
#undef MSA_GEMM_READ_ONE

    // ---- epilogue: column maxima over the tile's real tokens (one
    // accumulator column block at a time: the scheduler barrier keeps the
    // reads of the accumulation registers from being hoisted all at once)
    const int64_t t_in = (qt * GB) % Tq_pad;
    const int real = (Tq - t_in < GB) ? int(Tq - t_in) : GB;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        __builtin_amdgcn_sched_barrier(0);
        float m = -INFINITY;
        if (real == GB) {
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int i = 0; i < 16; ++i) m = fmaxf(m, acc[a][b][i]);
        } else {
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = wm * 128 + a * 32 + (i / 4) * 8 + (lane / 32) * 4 + (i % 4);
                    m = (r < real) ? fmaxf(m, acc[a][b][i]) : m;
                }
        }
        m = fmaxf(m, __shfl_xor(m, 32));
        if (lane < 32) sMax[wm][wn * 128 + b * 32 + lane] = m;
    }
    __syncthreads();
    const int64_t n = ct * GB + tid;
    if (n < N) partial[qt * N + n] = fmaxf(sMax[0][tid], sMax[1][tid]) * inv_hq;
}

struct Plan {
    bool gemm;
    int bm, bn, tq_pad;
    int64_t q_pad, q_tiles, n_pad;
    size_t ub_bytes, partial_bytes, rn_bytes, kp_bytes;
};

// Tq == 1: rows are queries (32-row tiles for up to 32 queries, else 128).
// Tq a multiple of 256, or >= 1,024: the GEMM, each query padded to a multiple
// of 256 tokens (at most 20% padding).  Otherwise 128-row tiles for Tq > 32
// and 32-row tiles below, each query padded to a multiple of the tile.
Plan plan_for(int64_t B, int Tq, int Hkv, int64_t N) {
    Plan p;
    const int64_t Q = B * Tq;
    p.gemm = Tq > 1 && (Tq % GB == 0 || Tq >= 1024);
    if (p.gemm) {
        p.bm = p.bn = GB;
        p.tq_pad = int(ceil_div(int64_t(Tq), int64_t(GB)) * GB);
        p.q_pad = B * p.tq_pad;
        p.q_tiles = p.q_pad / GB;
        p.n_pad = ceil_div(N, int64_t(GB)) * GB;
        p.ub_bytes = align256(size_t(p.q_pad) * Hkv * 128 * 2);
        p.kp_bytes = align256(size_t(p.n_pad) * Hkv * 128 * 2);
        p.partial_bytes = align256(size_t(p.q_tiles) * N * 4);
        p.rn_bytes = 0;
        return p;
    }
    p.kp_bytes = 0;
    p.n_pad = N;
    p.bm = (Tq == 1) ? (Q <= 32 ? 32 : 128) : (Tq > 32 ? 128 : 32);
    p.bn = 128;
    if (Tq == 1) {
        p.tq_pad = 1;
        p.q_pad = ceil_div(Q, p.bm) * p.bm;
    } else {
        p.tq_pad = int(ceil_div(int64_t(Tq), int64_t(p.bm)) * p.bm);
        p.q_pad = B * p.tq_pad;
    }
    p.q_tiles = p.q_pad / p.bm;
    p.ub_bytes = align256(size_t(p.q_pad) * Hkv * 128 * 2);
    p.partial_bytes = (Tq == 1) ? 0 : align256(size_t(p.q_tiles) * N * 4);
    p.rn_bytes = (p.q_tiles > 1) ? align256(size_t(N) * Hkv * 4) : 0;   // norms computed once, shared by the query tiles
    return p;
}

}  // namespace

bool route_mfma_applicable(msa_dtype dt, int64_t B, int Tq, int Hkv, int D) {
    if (dt != MSA_BF16 || D != 128 || Hkv < 1) return false;
    return B * Tq > 4;                             // the streaming scan handles decode
}

bool route_mfma_preps_itself(const RouteArgs& a) {
    return route_mfma_applicable(a.dt, a.B, a.Tq, a.Hkv, a.D) && !plan_for(a.B, a.Tq, a.Hkv, a.N).gemm &&
           (reinterpret_cast<uintptr_t>(a.Qr) & 15u) == 0;
}

size_t route_mfma_workspace(msa_dtype dt, int64_t B, int Tq, int Hq, int Hkv, int D, int64_t N, int) {
    (void)Hq;
    if (!route_mfma_applicable(dt, B, Tq, Hkv, D)) return 0;
    const Plan p = plan_for(B, Tq, Hkv, N);
    return p.ub_bytes + p.partial_bytes + p.rn_bytes + p.kp_bytes;
}

hipError_t launch_route_mfma(const RouteArgs& a, const float* U, float* c, void* ws, hipStream_t st) {
    const Plan p = plan_for(a.B, a.Tq, a.Hkv, a.N);
    const int64_t Q = a.B * a.Tq;
    hipError_t err;
    if (p.gemm) {
        const int K = a.Hkv * 128, S = K / GK;
        u32x4* Up = static_cast<u32x4*>(ws);
        float* partial = reinterpret_cast<float*>(static_cast<char*>(ws) + p.ub_bytes);
        u32x4* Kp = reinterpret_cast<u32x4*>(static_cast<char*>(ws) + p.ub_bytes + p.partial_bytes);
        hipLaunchKernelGGL(route_u_pack, dim3(unsigned(ceil_div(p.q_pad * (K / 8), 256))), dim3(256), 0, st, U, a.B,
                           a.Tq, p.tq_pad, p.q_pad, K, Up);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(route_khat_pack, dim3(unsigned(ceil_div(p.n_pad * a.Hkv * 16, 256))), dim3(256), 0, st,
                           static_cast<const uint16_t*>(a.Krbar), a.N, p.n_pad, a.Hkv, Kp);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        const TileOrder ord = tile_order(p.q_tiles, p.n_pad / GB, 4, 8);
        err = launch_timed(route_gemm_kernel, dim3(unsigned(ord.blocks)), dim3(256), st, a.prof_start, a.prof_stop,
                           static_cast<const u32x4*>(Up), static_cast<const u32x4*>(Kp), a.N, S, a.Tq, p.tq_pad,
                           1.f / float(a.Hq), partial, ord);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(route_mfma_tokmax, dim3(unsigned(ceil_div(a.B * a.N, 256))), dim3(256), 0, st, partial,
                           a.N, int(p.tq_pad / GB), a.B, c);
        return hipGetLastError();
    }
    uint16_t* Ub = static_cast<uint16_t*>(ws);
    float* partial = reinterpret_cast<float*>(static_cast<char*>(ws) + p.ub_bytes);
    float* rn = reinterpret_cast<float*>(static_cast<char*>(ws) + p.ub_bytes + p.partial_bytes);
    const int64_t n_pad = p.q_pad * a.Hkv * 128;
    if (route_mfma_preps_itself(a)) {             // U is formed here, straight into the padded bf16 operand
        const int64_t items = p.q_pad * a.Hkv;
        int64_t blocks = ceil_div(items, int64_t(4));
        if (blocks > int64_t(a.num_cus) * 8) blocks = int64_t(a.num_cus) * 8;
        hipLaunchKernelGGL(route_prep_ub_kernel, dim3(unsigned(blocks < 1 ? 1 : blocks)), dim3(256), 0, st,
                           static_cast<const u32x4*>(a.Qr), a.B, a.Tq, p.tq_pad, items, a.Hq, a.Hkv,
                           reinterpret_cast<u32x4*>(Ub));
    } else {
        hipLaunchKernelGGL(u_to_bf16_kernel, dim3(unsigned(ceil_div(n_pad, 256))), dim3(256), 0, st, U, a.B, a.Tq,
                           p.tq_pad, a.Hkv * 128, n_pad, Ub);
    }
    err = hipGetLastError();
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
    const uint16_t* Ubc = Ub;
    const float* rnc = rn;
    if (p.bm == 32)
        err = p.rn_bytes ? launch_timed(route_mfma_kernel<32, 128, true>, grid, dim3(256), st, a.prof_start, a.prof_stop,
                                        Ubc, Q, Kr, a.N, a.Hkv, a.Tq, p.tq_pad, inv_hq, c, partial, ord, rnc)
                         : launch_timed(route_mfma_kernel<32, 128, false>, grid, dim3(256), st, a.prof_start, a.prof_stop,
                                        Ubc, Q, Kr, a.N, a.Hkv, a.Tq, p.tq_pad, inv_hq, c, partial, ord, rnc);
    else
        err = p.rn_bytes ? launch_timed(route_mfma_kernel<128, 128, true>, grid, dim3(256), st, a.prof_start, a.prof_stop,
                                        Ubc, Q, Kr, a.N, a.Hkv, a.Tq, p.tq_pad, inv_hq, c, partial, ord, rnc)
                         : launch_timed(route_mfma_kernel<128, 128, false>, grid, dim3(256), st, a.prof_start, a.prof_stop,
                                        Ubc, Q, Kr, a.N, a.Hkv, a.Tq, p.tq_pad, inv_hq, c, partial, ord, rnc);
    if (err != hipSuccess) return err;
    if (a.Tq > 1) {
        hipLaunchKernelGGL(route_mfma_tokmax, dim3(unsigned(ceil_div(a.B * a.N, 256))), dim3(256), 0, st, partial,
                           a.N, int(p.tq_pad / p.bm), a.B, c);
        err = hipGetLastError();
    }
    return err;
}

}  // namespace msa
