// Stage 3 on the matrix cores: prefill (many query tokens) GQA attention over
// [selected K̄/V̄ ; local K/V] with global RoPE and a causal local segment.
//
// Source: news.neo-ai.one MSA article, 全体設計 › アーキテクチャ (Fig. 2): the
// compressed K/V of the selected documents are concatenated with the query's
// local K/V; global RoPE shifts the query's start by k (background -> query
// -> generation).  Same key space, positions and mask as attn.hip.
//
// attn_prefill_kernel: a workgroup (4 waves) owns 128 query tokens of one query
// head h (KV head h / G); wave w owns tokens 32w .. 32w+31.  Keys are taken 64
// at a time: the memory rows first, then the local rows up to the last token
// the tile can see.  Per key tile:
//   * the loader puts K (local rows rotated at q_offset + j in fp32, then
//     rounded to bf16) in LDS row-major, and V transposed (d-major), so both
//     matrix-core operands are read with 16- or 8-byte LDS loads;
//   * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 (two 32-key tiles, 8 k-steps
//     over d), so each lane holds the 32 scores of one query token;
//   * masking, an online softmax in the log2 domain (the scale 1/sqrt(d) and
//     log2(e) are folded into Q before its bf16 rounding), P rounded to bf16;
//   * O += P . V: the 16 keys of a k-step are taken in the order the score
//     accumulator already holds them (any order is a valid contraction order,
//     as long as P and V agree), so P needs no shuffle; V fragments are two
//     8-byte reads of the transposed tile.
// Per-query rescale factors and row sums reach the output layout (query per
// register) with one lane shuffle each.
#include "attn_mfma.hpp"

namespace msa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BQ = 128, BK = 64, DH = 128;
constexpr int KST = DH + 8;      // K / Q tile row stride (bf16)
constexpr int VST = BK + 4;      // transposed V tile row stride (bf16), keeps 8-byte alignment
constexpr int kSmem = (BQ * KST > BK * KST + DH * VST) ? BQ * KST : BK * KST + DH * VST;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return uint32_t(f32_to_bf16(a)) | (uint32_t(f32_to_bf16(b)) << 16);
}

__global__ __launch_bounds__(256) void attn_prefill_kernel(
    const uint16_t* __restrict__ Q, int Tq, int Hq, int hkv, const uint16_t* __restrict__ KVmem,
    const int64_t* __restrict__ mem_off, int64_t cap, int64_t max_rows, const uint16_t* __restrict__ Kl,
    const uint16_t* __restrict__ Vl, int L, int q_offset, float qscale, const float2* __restrict__ rope,
    int max_pos, uint16_t* __restrict__ O) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[kSmem];
    uint16_t* sQ = smem;                 // prologue only
    uint16_t* sK = smem;                 // key loop (aliases sQ)
    uint16_t* sVt = smem + BK * KST;

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int qt = int(gridDim.x) - 1 - int(blockIdx.x);          // longest (latest) tiles first
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int G = Hq / hkv, g = h / G;
    const int i0 = qt * BQ;
    const int64_t kv_row = int64_t(hkv) * DH;

    // ---- rotated, scaled query rows of this tile -> LDS (bf16)
    for (int idx = tid; idx < BQ * (DH / 2); idx += 256) {
        const int r = idx / (DH / 2), c = idx % (DH / 2);
        const int i = i0 + r;
        float y1 = 0.f, y2 = 0.f;
        if (i < Tq) {
            int pos = q_offset + (L - Tq) + i;
            pos = pos < max_pos ? pos : max_pos - 1;
            const int64_t qb = ((b * Tq + i) * Hq + h) * DH;
            const float x1 = bf16_to_f32(Q[qb + c]), x2 = bf16_to_f32(Q[qb + c + DH / 2]);
            const float2 cs = rope[int64_t(pos) * (DH / 2) + c];
            y1 = (x1 * cs.x - x2 * cs.y) * qscale;
            y2 = (x2 * cs.x + x1 * cs.y) * qscale;
        }
        sQ[r * KST + c] = f32_to_bf16(y1);
        sQ[r * KST + c + DH / 2] = f32_to_bf16(y2);
    }
    __syncthreads();
    bf16x8 qf[8];                        // B operand of S^T: d = 16 ks + 8 (lane/32) + e, query = lane % 32
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
        qf[ks] = *reinterpret_cast<const bf16x8*>(sQ + (wave * 32 + lane % 32) * KST + ks * 16 + (lane / 32) * 8);
    __syncthreads();

    // ---- key space of this tile
    int64_t r0 = mem_off[b], r1 = mem_off[b + 1];
    r0 = r0 < 0 ? 0 : (r0 > cap ? cap : r0);
    r1 = r1 < r0 ? r0 : (r1 > cap ? cap : r1);
    if (r1 - r0 > max_rows) r1 = r0 + max_rows;
    const int64_t M = r1 - r0;
    const int last_q = (i0 + BQ < Tq ? i0 + BQ : Tq) - 1;
    const int64_t jmax = int64_t(L - Tq) + last_q;                 // last local key any token here sees
    const int64_t total = M + jmax + 1;
    const int n_tiles = int((total + BK - 1) / BK);
    const int qi = i0 + wave * 32 + lane % 32;                      // this lane's query token
    const int64_t lim = int64_t(L - Tq) + qi;                       // local key j visible iff j <= lim

    float m_run = -INFINITY, l_run = 0.f;
    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;

    for (int t = 0; t < n_tiles; ++t) {
        const int64_t k0 = int64_t(t) * BK;
        // ---- K tile: 8 threads per key, each a pair of 16-byte halves (i, i + 64)
        for (int idx = tid; idx < BK * 8; idx += 256) {
            const int kk = idx / 8, c = (idx % 8) * 8;
            const int64_t key = k0 + kk;
            u32x4 w1 = {0u, 0u, 0u, 0u}, w2 = {0u, 0u, 0u, 0u};
            if (key < M) {
                const uint16_t* row = KVmem + ((r0 + key) * 2) * kv_row + int64_t(g) * DH;
                w1 = *reinterpret_cast<const u32x4*>(row + c);
                w2 = *reinterpret_cast<const u32x4*>(row + c + DH / 2);
            } else if (key < total) {
                const int64_t j = key - M;
                const uint16_t* row = Kl + ((b * L + j) * hkv + g) * DH;
                const u32x4 x1 = *reinterpret_cast<const u32x4*>(row + c);
                const u32x4 x2 = *reinterpret_cast<const u32x4*>(row + c + DH / 2);
                int pos = q_offset + int(j);
                pos = pos < max_pos ? pos : max_pos - 1;
                const float2* cs = rope + int64_t(pos) * (DH / 2) + c;
                float a[8], bb[8], y1[8], y2[8];
                a[0] = bf16_lo(x1.x); a[1] = bf16_hi(x1.x); a[2] = bf16_lo(x1.y); a[3] = bf16_hi(x1.y);
                a[4] = bf16_lo(x1.z); a[5] = bf16_hi(x1.z); a[6] = bf16_lo(x1.w); a[7] = bf16_hi(x1.w);
                bb[0] = bf16_lo(x2.x); bb[1] = bf16_hi(x2.x); bb[2] = bf16_lo(x2.y); bb[3] = bf16_hi(x2.y);
                bb[4] = bf16_lo(x2.z); bb[5] = bf16_hi(x2.z); bb[6] = bf16_lo(x2.w); bb[7] = bf16_hi(x2.w);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float2 r = cs[e];
                    y1[e] = a[e] * r.x - bb[e] * r.y;
                    y2[e] = bb[e] * r.x + a[e] * r.y;
                }
                w1 = u32x4{pack2(y1[0], y1[1]), pack2(y1[2], y1[3]), pack2(y1[4], y1[5]), pack2(y1[6], y1[7])};
                w2 = u32x4{pack2(y2[0], y2[1]), pack2(y2[2], y2[3]), pack2(y2[4], y2[5]), pack2(y2[6], y2[7])};
            }
            *reinterpret_cast<u32x4*>(sK + kk * KST + c) = w1;
            *reinterpret_cast<u32x4*>(sK + kk * KST + c + DH / 2) = w2;
        }
        // ---- V tile, transposed: sVt[d][key]
        for (int idx = tid; idx < BK * 16; idx += 256) {
            const int kk = idx / 16, c = (idx % 16) * 8;
            const int64_t key = k0 + kk;
            u32x4 w = {0u, 0u, 0u, 0u};
            if (key < M) w = *reinterpret_cast<const u32x4*>(KVmem + ((r0 + key) * 2 + 1) * kv_row + int64_t(g) * DH + c);
            else if (key < total) w = *reinterpret_cast<const u32x4*>(Vl + ((b * L + (key - M)) * hkv + g) * DH + c);
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sVt[(c + 2 * e) * VST + kk] = uint16_t(ww[e] & 0xFFFFu);
                sVt[(c + 2 * e + 1) * VST + kk] = uint16_t(ww[e] >> 16);
            }
        }
        __syncthreads();

        // ---- S^T for two 32-key sub-tiles: rows = keys, columns = this wave's queries
        f32x16 s[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[tt][i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + (tt * 32 + lane % 32) * KST + ks * 16 + (lane / 32) * 8);
                s[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[tt], 0, 0, 0);
            }

        // ---- mask and online softmax (log2 domain); lanes l and l+32 share a query
        float mt = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int64_t key = k0 + tt * 32 + (i / 4) * 8 + (lane / 32) * 4 + (i % 4);
                const bool vis = key < total && (key < M || (key - M) <= lim) && qi < Tq;
                s[tt][i] = vis ? s[tt][i] : -INFINITY;
                mt = fmaxf(mt, s[tt][i]);
            }
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);
        const bool none = (m_new == -INFINITY);
        const float corr = (m_run == -INFINITY) ? (none ? 1.f : 0.f) : __builtin_amdgcn_exp2f(m_run - m_new);
        float rs = 0.f;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = (none || s[tt][i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[tt][i] - m_new);
                s[tt][i] = p;
                rs += p;
            }
        rs += __shfl_xor(rs, 32);
        l_run = l_run * corr + rs;
        m_run = m_new;

        // ---- rescale O: register i holds query (i/4)*8 + (lane/32)*4 + i%4 of this wave
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float f = __shfl(corr, (i / 4) * 8 + (lane / 32) * 4 + (i % 4));
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) o[dt][i] *= f;
        }

        // ---- O += P . V over 4 k-steps of 16 keys, in accumulator order
        // operands are assembled as packed dwords and bit-cast whole (element-wise
        // inserts of 16-bit lanes into the operand vector are not used)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int tt = ks / 2, sp = ks % 2;
            const u32x4 pw = {pack2(s[tt][sp * 8 + 0], s[tt][sp * 8 + 1]), pack2(s[tt][sp * 8 + 2], s[tt][sp * 8 + 3]),
                              pack2(s[tt][sp * 8 + 4], s[tt][sp * 8 + 5]), pack2(s[tt][sp * 8 + 6], s[tt][sp * 8 + 7])};
            const bf16x8 pa = __builtin_bit_cast(bf16x8, pw);
            const int ka = tt * 32 + sp * 16 + (lane / 32) * 4;     // keys ka..ka+3 and ka+8..ka+11
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const int d = dt * 32 + lane % 32;
                const u32x2 lo = *reinterpret_cast<const u32x2*>(sVt + d * VST + ka);
                const u32x2 hi = *reinterpret_cast<const u32x2*>(sVt + d * VST + ka + 8);
                const u32x4 vw = {lo.x, lo.y, hi.x, hi.y};
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, __builtin_bit_cast(bf16x8, vw), o[dt], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // ---- normalise and store
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int qr = (i / 4) * 8 + (lane / 32) * 4 + (i % 4);
        const float lsum = __shfl(l_run, qr);
        const int qtok = i0 + wave * 32 + qr;
        if (qtok < Tq) {
            const float inv = 1.f / lsum;
            const int64_t ob = ((b * Tq + qtok) * Hq + h) * DH;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) O[ob + dt * 32 + lane % 32] = f32_to_bf16(o[dt][i] * inv);
        }
    }
}

}  // namespace

bool attn_mfma_applicable(const AttnArgs& a) {
    return a.dt == MSA_BF16 && a.D == DH && a.Tq >= 64;
}

size_t attn_mfma_workspace(msa_dtype, int64_t, int, int, int, int, int64_t, int) { return 0; }

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t st) {
    const dim3 grid(unsigned(ceil_div(a.Tq, BQ)), unsigned(a.Hq), unsigned(a.B));
    hipLaunchKernelGGL(attn_prefill_kernel, grid, dim3(256), 0, st, static_cast<const uint16_t*>(a.Q), a.Tq,
                       a.Hq, a.Hkv, static_cast<const uint16_t*>(a.KVmem), a.mem_off, a.mem_rows_cap, a.max_rows,
                       static_cast<const uint16_t*>(a.K_local), static_cast<const uint16_t*>(a.V_local), a.L,
                       a.q_offset, a.scale * kLog2e, a.rope_cs, a.max_pos, static_cast<uint16_t*>(a.O));
    return hipGetLastError();
}

}  // namespace msa
