// Backward of stage 3 on the matrix cores: the gradients of the GQA attention
// over [selected K̄/V̄ ; local K/V] with respect to Q, the memory rows K̄ and V̄,
// and the local K and V, given dO and the row log-sum-exp the forward saved.
//
// Sources: ruixiangma.github.io blog, 训练策略 (the generation loss trains the
// model through this attention, beside the auxiliary routing loss);
// github-eval-reports review of MSA, 核心能力 › 端到端可训练框架 (retrieval and
// generation form one differentiable loop).  The forward differentiated is that
// of news.neo-ai.one MSA article, 全体設計 › アーキテクチャ (Fig. 2), with the
// key space, positions and mask of attn.hip.
//
// With P the softmax of a query row, dP_j = dO . v_j, D = dO . O and
// dS_j = P_j (dP_j - D): dV_j = sum_i P_ij dO_i, dk~_j = scale sum_i dS_ij q~_i
// and dq~_i = scale sum_j dS_ij k~_j, where ~ marks rotated vectors; the
// gradients of Q and of the local keys are the rotated ones turned back by
// their RoPE angle (the rotation is orthogonal), memory keys take theirs as
// they are.  P is recomputed from the saved log-sum-exp, so nothing of size
// (tokens x keys) is stored.
//
// Four kernels.
//
//   bwd_prep_q  per (b, query head, 32 query rows): scale * rotated Q and dO,
//               each as a row tile (32 x 128) and as a transposed tile
//               (128 x 32), bf16, 8 KB each, plus the rows' lse * log2(e)
//               (+inf past Tq, so those rows get P = 0) and D = dO . O.
//   bwd_prep_k  per (b, KV head, 32 keys): the key space as the forward sees
//               it (memory rows as stored, local keys rotated at q_offset + j,
//               zeros past the end) as a row tile and a transposed tile, and V
//               as a row tile.
//   Row tiles hold 16-byte unit u of row r at r*16 + (u ^ (r & 15)); transposed
//   tiles hold the 8-byte unit u (columns 4u .. 4u+3) of row c at
//   c*8 + (u ^ ((c >> 1) & 7)).  With these swizzles every matrix-core operand
//   read below hits distinct LDS banks across each 16 lanes, and a tile is
//   staged into LDS as one flat 8 KB copy.
//
//   bwd_dkdv    a workgroup (8 waves) owns 128 keys of one (b, KV head); wave
//               w takes keys 32 (w % 4) .. +31, waves 0..3 forming dV and waves
//               4..7 dK, so a SIMD runs one wave of each role and each wave
//               keeps only its accumulators (32 x 128 fp32) and one operand
//               (K or V of its keys) in registers.  The workgroup walks the
//               query tiles that can see its keys in pairs, from the last pair
//               down, the G heads of a pair together (so the workgroups of one
//               KV head running at the same time read the same tiles, from
//               L2); a pair is staged in LDS by direct global->LDS copies one
//               pair ahead.  Per pair, in two phases split by a barrier: the
//               dV wave forms S = Q K^T of both tiles on
//               v_mfma_f32_32x32x16_bf16 (two interleaved chains, keys along
//               the accumulator's columns), P = exp2(S log2 e - lse), and hands
//               P (bf16) to the dK wave of the same keys through LDS while that
//               wave forms dP = dO V^T; then the dV wave runs dV += P^T dO and
//               the dK wave dS = P (dP - D), dK += dS^T Q, against the
//               transposed tiles.  A k-step takes its 16 queries in the order
//               the accumulator holds them ({16k + 4u .. +3, 16k + 8 + 4u ..
//               +3} for lane half u), which is two 8-byte units of a transposed
//               row, so P and dS need no shuffle.
//   bwd_dq      a workgroup (4 waves) owns 32-token query tiles of up to four
//               query heads of one KV group (for G < 4, several tiles of each
//               head), so every staged key tile serves all four waves.  Each
//               wave keeps its Q and dO as operands and walks the key tiles its
//               tokens can see: S^T = K Q^T and dP^T = V dO^T (tokens along the
//               columns), then dQ^T += K^T dS^T.
// dQ is computed apart from dK/dV (S and dP again), so that no gradient is
// accumulated with atomics: every output element is written once, in bf16,
// and the result does not depend on scheduling.  Workgroups take the
// heaviest tiles first; when B * Hkv is a multiple of the 8 XCDs, all
// workgroups of one (b, KV head) share an XCD and its L2.
#include "launch.hpp"
#include "lds_dma.hpp"

namespace msa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int DH = 128;
constexpr int RB = 32;                       // rows (tokens or keys) per tile
constexpr int kTile = RB * DH / 8;           // 16-byte units of a tile: 512 (8 KB)
constexpr int kStat = 16;                    // 16-byte units of a query tile's statistics (64 floats)
constexpr int kKeysWg = 128;                 // keys per bwd_dkdv workgroup (4 waves x 32)
constexpr int kStageQ = 4 * kTile + kStat;   // one bwd_dkdv stage: Q, Q^T, dO, dO^T, statistics
constexpr int kStageK = 3 * kTile;           // one bwd_dq stage: K, K^T, V
constexpr int PST = DH + 8;                  // LDS staging row stride (bf16) of the prep kernels
constexpr float kLog2e = 1.4426950408889634f;

__host__ __device__ inline int row_unit(int r, int u) { return r * 16 + (u ^ (r & 15)); }
__host__ __device__ inline int tr_unit8(int c, int u) { return c * 8 + (u ^ ((c >> 1) & 7)); }

// Register i of a 32 x 32 accumulator holds this row of the lane's column.
__device__ __forceinline__ int acc_row(int i, int half) { return (i / 4) * 8 + half * 4 + (i % 4); }

__device__ __forceinline__ float elem(const u32x4& w, int e) {
    return (e & 1) ? bf16_hi(w[e / 2]) : bf16_lo(w[e / 2]);
}

__device__ __forceinline__ u32x4 pack8(const float* y) {
    return u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                 pack_bf16x2(y[6], y[7])};
}

// Rotates (x1, x2) = dimensions (c .. c+7, c+64 .. c+71) by the angle table row cs.
__device__ __forceinline__ void rotate8(const u32x4& x1, const u32x4& x2, const float2* cs, float mul,
                                        float* y1, float* y2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float a = elem(x1, e), bb = elem(x2, e);
        const float2 r = cs[e];
        y1[e] = (a * r.x - bb * r.y) * mul;
        y2[e] = (bb * r.x + a * r.y) * mul;
    }
}

// The 32 x 128 tile staged in s (rows of PST) written transposed: 128 rows of
// 8 units, each unit 4 consecutive columns.
__device__ __forceinline__ void write_transposed(const uint16_t* s, u32x4* dst, int tid) {
    uint2* d8 = reinterpret_cast<uint2*>(dst);
    for (int k = tid; k < DH * 8; k += 256) {
        const int c = k / 8, u = k % 8;
        const uint32_t a0 = uint32_t(s[(4 * u) * PST + c]) | (uint32_t(s[(4 * u + 1) * PST + c]) << 16);
        const uint32_t a1 = uint32_t(s[(4 * u + 2) * PST + c]) | (uint32_t(s[(4 * u + 3) * PST + c]) << 16);
        d8[tr_unit8(c, u)] = make_uint2(a0, a1);
    }
}

__global__ __launch_bounds__(256) void bwd_prep_q_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
    const float* __restrict__ lse, int Tq, int Hq, int L, int q_offset, float scale,
    const float2* __restrict__ rope, int max_pos, int nqb, u32x4* __restrict__ QB, u32x4* __restrict__ QT,
    u32x4* __restrict__ OB, u32x4* __restrict__ OT, float* __restrict__ ST) {
    __shared__ __attribute__((aligned(16))) uint16_t sq[RB * PST];
    __shared__ __attribute__((aligned(16))) uint16_t so[RB * PST];
    const int tid = threadIdx.x;
    const int qb = blockIdx.x, h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int64_t tile = (b * Hq + h) * nqb + qb;
    const int r = tid / 8, u = tid % 8;              // row r, dimensions 8u .. 8u+7 and 64 + 8u ..
    const int q = qb * RB + r;
    const bool valid = q < Tq;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    u32x4 w1 = zero, w2 = zero, o1 = zero, o2 = zero;
    float dsum = 0.f;
    if (valid) {
        const int64_t base = ((b * Tq + q) * Hq + h) * DH + 8 * u;
        const u32x4 x1 = *reinterpret_cast<const u32x4*>(Q + base);
        const u32x4 x2 = *reinterpret_cast<const u32x4*>(Q + base + DH / 2);
        int pos = q_offset + (L - Tq) + q;
        pos = pos < max_pos ? pos : max_pos - 1;
        float y1[8], y2[8];
        rotate8(x1, x2, rope + int64_t(pos) * (DH / 2) + 8 * u, scale, y1, y2);
        w1 = pack8(y1);
        w2 = pack8(y2);
        o1 = *reinterpret_cast<const u32x4*>(dO + base);
        o2 = *reinterpret_cast<const u32x4*>(dO + base + DH / 2);
        const u32x4 p1 = *reinterpret_cast<const u32x4*>(O + base);
        const u32x4 p2 = *reinterpret_cast<const u32x4*>(O + base + DH / 2);
#pragma unroll
        for (int e = 0; e < 8; ++e) dsum += elem(o1, e) * elem(p1, e) + elem(o2, e) * elem(p2, e);
    }
    dsum = group_sum<8>(dsum);
    QB[tile * kTile + row_unit(r, u)] = w1;
    QB[tile * kTile + row_unit(r, u + 8)] = w2;
    OB[tile * kTile + row_unit(r, u)] = o1;
    OB[tile * kTile + row_unit(r, u + 8)] = o2;
    *reinterpret_cast<u32x4*>(sq + r * PST + 8 * u) = w1;
    *reinterpret_cast<u32x4*>(sq + r * PST + DH / 2 + 8 * u) = w2;
    *reinterpret_cast<u32x4*>(so + r * PST + 8 * u) = o1;
    *reinterpret_cast<u32x4*>(so + r * PST + DH / 2 + 8 * u) = o2;
    if (u == 0) {
        ST[tile * 64 + r] = valid ? lse[(b * Tq + q) * Hq + h] * kLog2e : INFINITY;
        ST[tile * 64 + 32 + r] = valid ? dsum : 0.f;
    }
    __syncthreads();
    write_transposed(sq, QT + tile * kTile, tid);
    write_transposed(so, OT + tile * kTile, tid);
}

__global__ __launch_bounds__(256) void bwd_prep_k_kernel(
    const uint16_t* __restrict__ KVmem, const int64_t* __restrict__ mem_off, int64_t cap, int64_t max_rows,
    const uint16_t* __restrict__ Kl, const uint16_t* __restrict__ Vl, int L, int hkv, int q_offset,
    const float2* __restrict__ rope, int max_pos, int nkb, u32x4* __restrict__ KB, u32x4* __restrict__ KT,
    u32x4* __restrict__ VB) {
    __shared__ __attribute__((aligned(16))) uint16_t sk[RB * PST];
    const int tid = threadIdx.x;
    const int kb = blockIdx.x, g = blockIdx.y;
    const int64_t b = blockIdx.z;
    int64_t r0, M;
    mem_range(mem_off, b, cap, max_rows, r0, M);
    const int64_t n_keys = M + L;
    const int64_t tile = (b * hkv + g) * nkb + kb;
    const int r = tid / 8, u = tid % 8;
    const int64_t key = int64_t(kb) * RB + r;
    const int64_t kv_row = int64_t(hkv) * DH;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    u32x4 w1 = zero, w2 = zero, v1 = zero, v2 = zero;
    if (key < M) {
        const uint16_t* row = KVmem + ((r0 + key) * 2) * kv_row + int64_t(g) * DH + 8 * u;
        w1 = *reinterpret_cast<const u32x4*>(row);
        w2 = *reinterpret_cast<const u32x4*>(row + DH / 2);
        v1 = *reinterpret_cast<const u32x4*>(row + kv_row);
        v2 = *reinterpret_cast<const u32x4*>(row + kv_row + DH / 2);
    } else if (key < n_keys) {
        const int64_t j = key - M;
        const int64_t base = ((b * L + j) * hkv + g) * DH + 8 * u;
        const u32x4 x1 = *reinterpret_cast<const u32x4*>(Kl + base);
        const u32x4 x2 = *reinterpret_cast<const u32x4*>(Kl + base + DH / 2);
        int pos = q_offset + int(j);
        pos = pos < max_pos ? pos : max_pos - 1;
        float y1[8], y2[8];
        rotate8(x1, x2, rope + int64_t(pos) * (DH / 2) + 8 * u, 1.f, y1, y2);
        w1 = pack8(y1);
        w2 = pack8(y2);
        v1 = *reinterpret_cast<const u32x4*>(Vl + base);
        v2 = *reinterpret_cast<const u32x4*>(Vl + base + DH / 2);
    }
    KB[tile * kTile + row_unit(r, u)] = w1;
    KB[tile * kTile + row_unit(r, u + 8)] = w2;
    VB[tile * kTile + row_unit(r, u)] = v1;
    VB[tile * kTile + row_unit(r, u + 8)] = v2;
    *reinterpret_cast<u32x4*>(sk + r * PST + 8 * u) = w1;
    *reinterpret_cast<u32x4*>(sk + r * PST + DH / 2 + 8 * u) = w2;
    __syncthreads();
    write_transposed(sk, KT + tile * kTile, tid);
}

// 8 bf16 of a transposed tile for a k-step: columns {16kk + 4half .. +3,
// 16kk + 8 + 4half .. +3} of row c, i.e. the accumulator's order of its rows.
__device__ __forceinline__ bf16x8 tr_operand(const u32x4* tile, int c, int kk, int half) {
    const uint2* t8 = reinterpret_cast<const uint2*>(tile);
    const uint2 lo = t8[tr_unit8(c, 4 * kk + half)];
    const uint2 hi = t8[tr_unit8(c, 4 * kk + 2 + half)];
    return __builtin_bit_cast(bf16x8, (u32x4{lo.x, lo.y, hi.x, hi.y}));
}

__device__ __forceinline__ bf16x8 pack_operand(const float* v) {
    return __builtin_bit_cast(bf16x8, pack8(v));
}

__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(
    const u32x4* __restrict__ QB, const u32x4* __restrict__ QT, const u32x4* __restrict__ OB,
    const u32x4* __restrict__ OT, const u32x4* __restrict__ ST, const u32x4* __restrict__ KB,
    const u32x4* __restrict__ VB, const int64_t* __restrict__ mem_off, int64_t cap, int64_t max_rows, int Tq,
    int Hq, int hkv, int L, int q_offset, const float2* __restrict__ rope, int max_pos, int nqb, int nkb,
    int64_t B, uint16_t* __restrict__ dKVmem, uint16_t* __restrict__ dKl, uint16_t* __restrict__ dVl) {
    // two stages of a tile pair, then P of the pair as packed bf16 operands
    // ([4 quarters][2 tiles][2 operands][64 lanes])
    __shared__ __attribute__((aligned(16))) u32x4 sbuf[2 * 2 * kStageQ + 4 * 2 * 2 * kWave];
    const int64_t n_bg = B * hkv;
    const int kt = int(blockIdx.x / n_bg);          // key tiles in order: the first (heaviest) first
    const int64_t bg = blockIdx.x % n_bg;
    const int64_t b = bg / hkv;
    const int g = int(bg % hkv);
    const int tid = threadIdx.x, lane = tid % kWave, half = lane / 32;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const bool kside = wave >= 4;                   // waves 4..7 form dK, waves 0..3 dV
    const int kq = wave % 4;                        // the wave's quarter of the 128 keys
    int64_t r0, M;
    mem_range(mem_off, b, cap, max_rows, r0, M);
    const int64_t n_keys = M + L;
    const int64_t k0 = int64_t(kt) * kKeysWg;
    if (k0 >= n_keys) return;                       // the whole workgroup: past this query's keys
    const int G = Hq / hkv;
    const int64_t shift = M + (L - Tq);             // token i sees keys 0 .. shift + i
    const int qb0 = k0 <= shift ? 0 : int((k0 - shift) / RB);   // the first query tile seeing the keys
    // the walk: pairs of query tiles (nqb-1, nqb-2), (nqb-3, nqb-4), ... down to
    // qb0, the G heads of a pair together
    const int n_it = G * ((nqb - qb0 + 1) / 2);
    const int64_t kw0 = k0 + 32 * kq;               // the wave's first key
    const int qbw = kw0 <= shift ? 0 : int((kw0 - shift) / RB);   // the wave's first query tile
    const int wave_its = qbw > nqb - 1 ? 0 : G * ((nqb - 1 - qbw) / 2 + 1);   // pairs whose first tile it sees
    const int64_t kcol = kw0 + lane % 32;           // this lane's key (a column of S)

    // the wave's 32 keys as B operands: K in the dV role (for S), V in the dK
    // role (for dP)
    bf16x8 kvf[8];
    {
        const int64_t tk = (bg * nkb + kt * 4 + kq) * kTile;
        const u32x4* src = kside ? VB : KB;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) kvf[ks] = __builtin_bit_cast(bf16x8, src[tk + row_unit(lane % 32, 2 * ks + half)]);
    }
    f32x16 acc[4];                                  // dV (waves 0..3) or dK (waves 4..7)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[n][i] = 0.f;

    const uint32_t lds0 = lds_addr(sbuf);
    const int64_t qbase = (b * Hq + int64_t(g) * G) * nqb;
    int hh_c = 0, qa_c = nqb - 1;                   // cursor of the next pair to copy
    auto dma = [&](int it) {
        const uint32_t sb = lds0 + uint32_t(it & 1) * 2 * kStageQ * 16;
        const u32x4* srcs[4] = {QB, QT, OB, OT};
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int qb = qa_c - t;
            if (qb < qb0) break;                    // the last pair may hold one tile
            const int64_t qt = qbase + int64_t(hh_c) * nqb + qb;
            const uint32_t st = sb + uint32_t(t) * kStageQ * 16;
            if (wave == t && lane < kStat)
                lds_copy16(ST + qt * kStat + lane, __builtin_amdgcn_readfirstlane(st + 4 * kTile * 16));
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
                lds_copy16(srcs[tt] + qt * kTile + wave * 64 + lane,
                           __builtin_amdgcn_readfirstlane(st + (tt * kTile + wave * 64) * 16));
        }
        if (++hh_c == G) {
            hh_c = 0;
            qa_c -= 2;
        }
    };
    u32x4* pbuf = sbuf + 2 * 2 * kStageQ + kq * 2 * 2 * kWave;   // this quarter's P: [2 tiles][2 operands][64]

    // P (or dS) of one tile from its scores, keys past a token's causal edge
    // masked only on tiles that cross the wave's keys (rows past Tq have
    // lse = +inf, so P = 0 there anyway)
    auto probs = [&](const f32x16& sc, const float* sst, int i0, float* p) {
        int64_t need = kcol - shift - i0;           // the token row from which this lane's key is visible
        need = need < -1 ? -1 : (need > RB ? RB : need);
        const int thr = int(need) - 4 * half;       // visible iff (i/4)*8 + i%4 >= thr
        const bool full = shift + i0 >= kw0 + 31;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 l4 = *reinterpret_cast<const float4*>(sst + 8 * j + 4 * half);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * j + e;
                float pv = __builtin_amdgcn_exp2f(sc[i] * kLog2e - lv[e]);
                if (!full) pv = ((i / 4) * 8 + (i % 4) >= thr) ? pv : 0.f;
                p[i] = pv;
            }
        }
    };

    // Per pair, in two phases split by a barrier: the dV waves form S and P of
    // both tiles (two interleaved chains) and hand P to the dK waves of the
    // same keys through LDS while those form dP; then the dV waves run
    // dV += P^T dO and the dK waves dS = P (dP - D), dK += dS^T Q.  S and the
    // exponentials are computed once; each wave runs 32 products per pair.
    dma(0);
    int hh = 0, ia = (nqb - 1) * RB;                // head and first token of the pair's first tile
    for (int it = 0; it < n_it; ++it) {
        MSA_WAIT_VMCNT(0);
        __syncthreads();                            // pair it in LDS; every wave done with pair it - 1
        if (it + 1 < n_it) dma(it + 1);
        const int iA = ia, iB = ia - RB;
        if (++hh == G) {
            hh = 0;
            ia -= 2 * RB;
        }
        const bool act = it < wave_its;
        const bool bv = act && iB >= qbw * RB;      // the pair's second tile exists and is seen
        const u32x4* sA = sbuf + (it & 1) * 2 * kStageQ;
        const u32x4* sB = sA + kStageQ;
        f32x16 xa, xb;                              // S (dV role) or dP (dK role) of the two tiles
        if (act) {
            const int off = kside ? 2 * kTile : 0;  // dO rows for dP, Q rows for S
#pragma unroll
            for (int i = 0; i < 16; ++i) xa[i] = xb[i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const bf16x8 a1 = __builtin_bit_cast(bf16x8, sA[off + row_unit(lane % 32, 2 * ks + half)]);
                xa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, kvf[ks], xa, 0, 0, 0);
                if (bv) {
                    const bf16x8 a2 = __builtin_bit_cast(bf16x8, sB[off + row_unit(lane % 32, 2 * ks + half)]);
                    xb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, kvf[ks], xb, 0, 0, 0);
                }
            }
        }
        if (!kside && act) {
            float p[16];
            probs(xa, reinterpret_cast<const float*>(sA + 4 * kTile), iA, p);
            pbuf[lane] = pack8(p);
            pbuf[kWave + lane] = pack8(p + 8);
            if (bv) {
                probs(xb, reinterpret_cast<const float*>(sB + 4 * kTile), iB, p);
                pbuf[2 * kWave + lane] = pack8(p);
                pbuf[3 * kWave + lane] = pack8(p + 8);
            }
        }
        __syncthreads();                            // P of the pair visible to the dK waves
        if (!act) continue;
        if (kside) {
            auto dk_tile = [&](const u32x4* sT, const f32x16& dp, const u32x4* pt) {
                const float* sst = reinterpret_cast<const float*>(sT + 4 * kTile);
                const u32x4 p0 = pt[lane], p1 = pt[kWave + lane];
                float ds[16];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float4 d4 = *reinterpret_cast<const float4*>(sst + 32 + 8 * j + 4 * half);
                    const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 4 * j + e;
                        ds[i] = elem(i < 8 ? p0 : p1, i % 8) * (dp[i] - dd[e]);
                    }
                }
                const bf16x8 da[2] = {pack_operand(ds), pack_operand(ds + 8)};
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int n = 0; n < 4; ++n)
                        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            da[kk], tr_operand(sT + kTile, n * 32 + lane % 32, kk, half), acc[n], 0, 0, 0);
            };
            dk_tile(sA, xa, pbuf);
            if (bv) dk_tile(sB, xb, pbuf + 2 * kWave);
        } else {
            auto dv_tile = [&](const u32x4* sT, const u32x4* pt) {
                const bf16x8 pa[2] = {__builtin_bit_cast(bf16x8, pt[lane]), __builtin_bit_cast(bf16x8, pt[kWave + lane])};
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int n = 0; n < 4; ++n)
                        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            pa[kk], tr_operand(sT + 3 * kTile, n * 32 + lane % 32, kk, half), acc[n], 0, 0, 0);
            };
            dv_tile(sA, pbuf);
            if (bv) dv_tile(sB, pbuf + 2 * kWave);
        }
    }

    // ---- store: register i holds key kw0 + acc_row(i, half), column n*32 + lane%32
    const int64_t kv_row = int64_t(hkv) * DH;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t key = kw0 + acc_row(i, half);
        if (key >= n_keys) continue;
        if (key < M) {
            uint16_t* row = dKVmem + ((r0 + key) * 2 + (kside ? 0 : 1)) * kv_row + int64_t(g) * DH + lane % 32;
#pragma unroll
            for (int n = 0; n < 4; ++n) row[n * 32] = f32_to_bf16(acc[n][i]);
        } else {
            const int64_t j = key - M;
            const int64_t base = ((b * L + j) * hkv + g) * DH + lane % 32;
            if (kside) {
                int pos = q_offset + int(j);
                pos = pos < max_pos ? pos : max_pos - 1;
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    const float2 cs = rope[int64_t(pos) * (DH / 2) + n * 32 + lane % 32];
                    const float y1 = acc[n][i], y2 = acc[n + 2][i];
                    dKl[base + n * 32] = f32_to_bf16(y1 * cs.x + y2 * cs.y);
                    dKl[base + n * 32 + DH / 2] = f32_to_bf16(y2 * cs.x - y1 * cs.y);
                }
            } else {
#pragma unroll
                for (int n = 0; n < 4; ++n) dVl[base + n * 32] = f32_to_bf16(acc[n][i]);
            }
        }
    }
}

__global__ __launch_bounds__(256) void bwd_dq_kernel(
    const u32x4* __restrict__ QB, const u32x4* __restrict__ OB, const float* __restrict__ ST,
    const u32x4* __restrict__ KB, const u32x4* __restrict__ KT, const u32x4* __restrict__ VB,
    const int64_t* __restrict__ mem_off, int64_t cap, int64_t max_rows, int Tq, int Hq, int hkv, int L,
    int q_offset, float scale, const float2* __restrict__ rope, int max_pos, int nqb, int nkb, int n_qg,
    int hsub, int64_t B, uint16_t* __restrict__ dQ) {
    __shared__ __attribute__((aligned(16))) u32x4 sbuf[2 * kStageK];
    const int G = Hq / hkv, G4 = G < 4 ? G : 4, qpw = 4 / G4;
    const int64_t n_bg = B * hkv;
    const int64_t n_inner = int64_t(hsub) * n_bg;
    const int rank = int(blockIdx.x / n_inner);
    const int64_t rest = blockIdx.x % n_inner;
    const int qg = n_qg - 1 - rank;                 // the last (heaviest) query tiles first
    const int sub = int(rest / n_bg);
    const int64_t bg = rest % n_bg;
    const int64_t b = bg / hkv;
    const int g = int(bg % hkv);
    const int tid = threadIdx.x, lane = tid % kWave, half = lane / 32;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int h = g * G + sub * G4 + wave % G4;
    const int qb = qg * qpw + wave / G4;
    const bool live = qb < nqb;
    const int iq = qb * RB + lane % 32;             // this lane's token (a column of S^T)
    int64_t r0, M;
    mem_range(mem_off, b, cap, max_rows, r0, M);
    const int64_t shift = M + (L - Tq);

    bf16x8 qf[8], of[8];
    float l2 = INFINITY, Dq = 0.f;
    if (live) {
        const int64_t qt = (b * Hq + h) * nqb + qb;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            qf[ks] = __builtin_bit_cast(bf16x8, QB[qt * kTile + row_unit(lane % 32, 2 * ks + half)]);
            of[ks] = __builtin_bit_cast(bf16x8, OB[qt * kTile + row_unit(lane % 32, 2 * ks + half)]);
        }
        l2 = ST[qt * 64 + lane % 32];
        Dq = ST[qt * 64 + 32 + lane % 32];
    } else {
        const bf16x8 z = __builtin_bit_cast(bf16x8, (u32x4{0u, 0u, 0u, 0u}));
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qf[ks] = of[ks] = z;
    }
    // key tiles: up to the last key the workgroup's (and the wave's) last token sees
    int last_q = (qg * qpw + qpw) * RB - 1;
    last_q = last_q < Tq - 1 ? last_q : Tq - 1;
    const int n_kb = int((shift + last_q) / RB) + 1;
    int wave_q = qb * RB + RB - 1;
    wave_q = wave_q < Tq - 1 ? wave_q : Tq - 1;
    const int wave_kb = live ? int((shift + wave_q) / RB) + 1 : 0;
    const bool wave_whole = live && qb * RB + RB - 1 < Tq;

    f32x16 dq[4];
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i) dq[n][i] = 0.f;

    const uint32_t lds0 = lds_addr(sbuf);
    auto dma = [&](int kb) {
        const int64_t t = (bg * nkb + kb) * kTile;
        const uint32_t sb = lds0 + uint32_t(kb & 1) * kStageK * 16;
        const u32x4* srcs[3] = {KB, KT, VB};
#pragma unroll
        for (int tt = 0; tt < 3; ++tt)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int piece = i * 4 + wave;
                lds_copy16(srcs[tt] + t + piece * 64 + lane,
                           __builtin_amdgcn_readfirstlane(sb + (tt * kTile + piece * 64) * 16));
            }
    };

    dma(0);
    for (int kb = 0; kb < n_kb; ++kb) {
        MSA_WAIT_VMCNT(0);
        __syncthreads();                            // tile kb in LDS; every wave done with tile kb - 1
        if (kb + 1 < n_kb) dma(kb + 1);
        if (kb >= wave_kb) continue;
        const u32x4* sK = sbuf + (kb & 1) * kStageK;
        const u32x4* sKT = sK + kTile;
        const u32x4* sV = sK + 2 * kTile;
        f32x16 st, dpt;
#pragma unroll
        for (int i = 0; i < 16; ++i) st[i] = dpt[i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const bf16x8 ka = __builtin_bit_cast(bf16x8, sK[row_unit(lane % 32, 2 * ks + half)]);
            st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], st, 0, 0, 0);
            const bf16x8 va = __builtin_bit_cast(bf16x8, sV[row_unit(lane % 32, 2 * ks + half)]);
            dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, of[ks], dpt, 0, 0, 0);
        }
        // every key of the tile visible to every token of the wave
        const bool full = wave_whole && shift + qb * RB >= int64_t(kb) * RB + RB - 1;
        const int64_t see = shift + iq;
        float ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float pv = __builtin_amdgcn_exp2f(st[i] * kLog2e - l2);
            if (!full && int64_t(kb) * RB + acc_row(i, half) > see) pv = 0.f;
            ds[i] = pv * (dpt[i] - Dq);
        }
        const bf16x8 db[2] = {pack_operand(ds), pack_operand(ds + 8)};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int n = 0; n < 4; ++n)
                dq[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(sKT, n * 32 + lane % 32, kk, half), db[kk],
                                                                 dq[n], 0, 0, 0);
    }

    // ---- store: register i of dq[n] holds dimension n*32 + acc_row(i, half) of token iq
    if (!live || iq >= Tq) return;
    int pos = q_offset + (L - Tq) + iq;
    pos = pos < max_pos ? pos : max_pos - 1;
    uint16_t* out = dQ + ((b * Tq + iq) * Hq + h) * DH;
    const float2* cs = rope + int64_t(pos) * (DH / 2);
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c0 = n * 32 + j * 8 + half * 4;       // dimensions c0 .. c0+3 and c0+64 ..
            float x1[4], x2[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float2 r = cs[c0 + e];
                const float y1 = dq[n][4 * j + e] * scale, y2 = dq[n + 2][4 * j + e] * scale;
                x1[e] = y1 * r.x + y2 * r.y;
                x2[e] = y2 * r.x - y1 * r.y;
            }
            *reinterpret_cast<uint2*>(out + c0) = make_uint2(pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3]));
            *reinterpret_cast<uint2*>(out + c0 + DH / 2) =
                make_uint2(pack_bf16x2(x2[0], x2[1]), pack_bf16x2(x2[2], x2[3]));
        }
}

struct BwdLayout {
    int nqb, nkb, n_kt;
    int64_t nq_tiles, nk_tiles;
    size_t q_bytes, st_bytes, k_bytes, total;
};

BwdLayout bwd_layout(int64_t B, int Tq, int Hq, int Hkv, int64_t max_rows, int L) {
    BwdLayout l;
    l.nqb = int(ceil_div(Tq, RB));
    const int64_t KP = ceil_div(max_rows + L, int64_t(kKeysWg)) * kKeysWg;
    l.nkb = int(KP / RB);
    l.n_kt = int(KP / kKeysWg);
    l.nq_tiles = B * Hq * l.nqb;
    l.nk_tiles = B * Hkv * l.nkb;
    l.q_bytes = align256(size_t(l.nq_tiles) * kTile * 16);
    l.st_bytes = align256(size_t(l.nq_tiles) * kStat * 16);
    l.k_bytes = align256(size_t(l.nk_tiles) * kTile * 16);
    l.total = 4 * l.q_bytes + l.st_bytes + 3 * l.k_bytes;
    return l;
}

}  // namespace

size_t attn_bwd_workspace(int64_t B, int Tq, int Hq, int Hkv, int64_t max_rows, int L) {
    return bwd_layout(B, Tq, Hq, Hkv, max_rows, L).total;
}

hipError_t launch_attn_bwd(const AttnBwdArgs& a, hipStream_t st) {
    const AttnArgs& f = a.f;
    if (f.B == 0 || f.Tq == 0) return hipSuccess;
    const BwdLayout l = bwd_layout(f.B, f.Tq, f.Hq, f.Hkv, f.max_rows, f.L);
    char* w = static_cast<char*>(f.ws);
    u32x4* QB = reinterpret_cast<u32x4*>(w);
    u32x4* QT = reinterpret_cast<u32x4*>(w + l.q_bytes);
    u32x4* OB = reinterpret_cast<u32x4*>(w + 2 * l.q_bytes);
    u32x4* OT = reinterpret_cast<u32x4*>(w + 3 * l.q_bytes);
    float* ST = reinterpret_cast<float*>(w + 4 * l.q_bytes);
    char* kw = w + 4 * l.q_bytes + l.st_bytes;
    u32x4* KB = reinterpret_cast<u32x4*>(kw);
    u32x4* KT = reinterpret_cast<u32x4*>(kw + l.k_bytes);
    u32x4* VB = reinterpret_cast<u32x4*>(kw + 2 * l.k_bytes);
    const uint16_t* KVmem = static_cast<const uint16_t*>(f.KVmem);

    hipLaunchKernelGGL(bwd_prep_q_kernel, dim3(unsigned(l.nqb), unsigned(f.Hq), unsigned(f.B)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(f.Q), static_cast<const uint16_t*>(f.O),
                       static_cast<const uint16_t*>(a.dO), a.lse, f.Tq, f.Hq, f.L, f.q_offset, f.scale, f.rope_cs,
                       f.max_pos, l.nqb, QB, QT, OB, OT, ST);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(bwd_prep_k_kernel, dim3(unsigned(l.nkb), unsigned(f.Hkv), unsigned(f.B)), dim3(256), 0, st,
                       KVmem, f.mem_off, f.mem_rows_cap, f.max_rows, static_cast<const uint16_t*>(f.K_local),
                       static_cast<const uint16_t*>(f.V_local), f.L, f.Hkv, f.q_offset, f.rope_cs, f.max_pos, l.nkb,
                       KB, KT, VB);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t n_bg = f.B * f.Hkv;
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3(unsigned(int64_t(l.n_kt) * n_bg)), dim3(512), 0, st, QB, QT, OB, OT,
                       reinterpret_cast<const u32x4*>(ST), KB, VB, f.mem_off, f.mem_rows_cap, f.max_rows, f.Tq,
                       f.Hq, f.Hkv, f.L, f.q_offset, f.rope_cs, f.max_pos, l.nqb, l.nkb, f.B,
                       static_cast<uint16_t*>(a.dKVmem), static_cast<uint16_t*>(a.dK_local),
                       static_cast<uint16_t*>(a.dV_local));
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int G = f.Hq / f.Hkv, G4 = G < 4 ? G : 4, qpw = 4 / G4, hsub = G / G4;
    const int n_qg = int(ceil_div(l.nqb, qpw));
    hipLaunchKernelGGL(bwd_dq_kernel, dim3(unsigned(int64_t(n_qg) * hsub * n_bg)), dim3(256), 0, st, QB, OB, ST, KB,
                       KT, VB, f.mem_off, f.mem_rows_cap, f.max_rows, f.Tq, f.Hq, f.Hkv, f.L, f.q_offset, f.scale,
                       f.rope_cs, f.max_pos, l.nqb, l.nkb, n_qg, hsub, f.B, static_cast<uint16_t*>(a.dQ));
    return hipGetLastError();
}

}  // namespace msa
