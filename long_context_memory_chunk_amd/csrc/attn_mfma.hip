// Stage 3 on the matrix cores: prefill (many query tokens) GQA attention over
// [selected K̄/V̄ ; local K/V] with global RoPE and a causal local segment.
//
// Source: news.neo-ai.one MSA article, 全体設計 › アーキテクチャ (Fig. 2): the
// compressed K/V of the selected documents are concatenated with the query's
// local K/V; global RoPE shifts the query's start by k (background -> query
// -> generation).  Same key space, positions and mask as attn.hip.
//
// Two kernels.
//
// attn_pack_kernel builds, once per (query b, KV head g), the key space in the
// layout the matrix cores read, in the workspace:
//   Kc[b][g][KP][d]  keys: the M_b memory rows as stored, then the L local keys
//                    rotated at q_offset + j (fp32, rounded once to bf16), then
//                    zeros up to KP (a multiple of 64);
//   Vt[b][g][KP/64][d][64]  values, transposed per 64-key tile, each 16-key
//                    group stored in the order the score accumulator holds its
//                    keys (see below), so a P.V operand is one 16-byte read.
// Every head of the group and every query tile reads these instead of
// rotating and transposing the same keys again.
//
// attn_prefill_kernel: a workgroup (4 waves) owns 128 query tokens of one query
// head h (KV head h / G); wave w owns tokens 32w .. 32w+31.  Keys are taken 64
// at a time up to the last local key the tile can see; each 64-key tile of Kc
// and Vt is 16 KB contiguous, copied to LDS with 16-byte accesses, and the next
// tile is fetched into registers while this one is used.  Per tile:
//   * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 (two 32-key tiles, 8 k-steps
//     over d), so each lane holds 32 scores of one query token (lanes l and
//     l + 32 share a token);
//   * masking only on tiles that cross a wave's causal edge; an online softmax
//     in the log2 domain (scale 1/sqrt(d) and log2(e) folded into Q before its
//     bf16 rounding).  The running max m is raised only when a score exceeds
//     it by more than 2^8: l and O are always scaled by the same m, so the
//     result is the same softmax, and the rescale of O is almost never taken;
//   * O += P . V: the 16 keys of a k-step are contracted in the order the score
//     accumulator holds them (lane half u holds keys {4u..4u+3, 8+4u..8+4u+3}),
//     which is the order Vt stores them in, so P needs no shuffle.
// Per-query rescale factors and row sums reach the output layout (query per
// register) with one lane shuffle each.
#include "attn_mfma.hpp"

namespace msa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BQ = 128, BK = 64, DH = 128;
constexpr int KST = DH + 8;      // K / Q tile row stride in LDS (bf16)
constexpr int VST = BK + 8;      // transposed V tile row stride in LDS (bf16)
constexpr int kSmemQ = BQ * KST;
constexpr int kSmemKV = BK * KST + DH * VST;
constexpr int kSmem = kSmemQ > kSmemKV ? kSmemQ : kSmemKV;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.f;     // raise the running max only past m + 8 (a factor 2^8)

// Memory rows of query b, clamped as in attn.hip.
__device__ __forceinline__ void mem_range(const int64_t* __restrict__ mem_off, int64_t b, int64_t cap,
                                          int64_t max_rows, int64_t& r0, int64_t& M) {
    int64_t a = mem_off[b], e = mem_off[b + 1];
    a = a < 0 ? 0 : (a > cap ? cap : a);
    e = e < a ? a : (e > cap ? cap : e);
    if (e - a > max_rows) e = a + max_rows;
    r0 = a;
    M = e - a;
}

// Position in a 16-key group -> key in that group (the score accumulator's order).
__device__ __forceinline__ int acc_key(int p) {
    const int u = p / 8, e = p % 8;
    return (e / 4) * 8 + 4 * u + (e % 4);
}

__global__ __launch_bounds__(256) void attn_pack_kernel(
    const uint16_t* __restrict__ KVmem, const int64_t* __restrict__ mem_off, int64_t cap, int64_t max_rows,
    const uint16_t* __restrict__ Kl, const uint16_t* __restrict__ Vl, int L, int hkv, int q_offset,
    const float2* __restrict__ rope, int max_pos, int64_t KP, uint16_t* __restrict__ Kc,
    uint16_t* __restrict__ Vt) {
    __shared__ __attribute__((aligned(16))) uint16_t sV[BK * KST];
    const int tid = threadIdx.x;
    const int tile = blockIdx.x, g = blockIdx.y;
    const int64_t b = blockIdx.z;
    int64_t r0, M;
    mem_range(mem_off, b, cap, max_rows, r0, M);
    const int64_t n_keys = M + L;
    const int64_t k0 = int64_t(tile) * BK;
    const int64_t kv_row = int64_t(hkv) * DH;
    const int64_t bg = b * hkv + g;

    // keys: 64 keys x 8 slot pairs (i, i + 64)
    for (int u = tid; u < BK * 8; u += 256) {
        const int kk = u / 8, c = (u % 8) * 8;
        const int64_t key = k0 + kk;
        u32x4 w1 = {0u, 0u, 0u, 0u}, w2 = {0u, 0u, 0u, 0u};
        if (key < M) {
            const uint16_t* row = KVmem + ((r0 + key) * 2) * kv_row + int64_t(g) * DH;
            w1 = *reinterpret_cast<const u32x4*>(row + c);
            w2 = *reinterpret_cast<const u32x4*>(row + c + DH / 2);
        } else if (key < n_keys) {
            const int64_t j = key - M;
            const uint16_t* row = Kl + ((b * L + j) * hkv + g) * DH;
            const u32x4 x1 = *reinterpret_cast<const u32x4*>(row + c);
            const u32x4 x2 = *reinterpret_cast<const u32x4*>(row + c + DH / 2);
            int pos = q_offset + int(j);
            pos = pos < max_pos ? pos : max_pos - 1;
            const float2* cs = rope + int64_t(pos) * (DH / 2) + c;
            float y1[8], y2[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t wa = x1[e / 2], wb = x2[e / 2];
                const float a = (e & 1) ? bf16_hi(wa) : bf16_lo(wa);
                const float bb = (e & 1) ? bf16_hi(wb) : bf16_lo(wb);
                const float2 r = cs[e];
                y1[e] = a * r.x - bb * r.y;
                y2[e] = bb * r.x + a * r.y;
            }
            w1 = u32x4{pack_bf16x2(y1[0], y1[1]), pack_bf16x2(y1[2], y1[3]), pack_bf16x2(y1[4], y1[5]),
                       pack_bf16x2(y1[6], y1[7])};
            w2 = u32x4{pack_bf16x2(y2[0], y2[1]), pack_bf16x2(y2[2], y2[3]), pack_bf16x2(y2[4], y2[5]),
                       pack_bf16x2(y2[6], y2[7])};
        }
        uint16_t* dst = Kc + (bg * KP + key) * DH;
        *reinterpret_cast<u32x4*>(dst + c) = w1;
        *reinterpret_cast<u32x4*>(dst + c + DH / 2) = w2;
    }

    // values: the 64 x 128 tile to LDS, then written transposed and permuted
    for (int u = tid; u < BK * 16; u += 256) {
        const int kk = u / 16, c = (u % 16) * 8;
        const int64_t key = k0 + kk;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (key < M) w = *reinterpret_cast<const u32x4*>(KVmem + ((r0 + key) * 2 + 1) * kv_row + int64_t(g) * DH + c);
        else if (key < n_keys) w = *reinterpret_cast<const u32x4*>(Vl + ((b * L + (key - M)) * hkv + g) * DH + c);
        *reinterpret_cast<u32x4*>(sV + kk * KST + c) = w;
    }
    __syncthreads();
    uint16_t* vt = Vt + ((bg * (KP / BK) + tile) * DH) * BK;
    for (int u = tid; u < DH * 8; u += 256) {
        const int d = u / 8, p0 = (u % 8) * 8;            // positions p0 .. p0+7 of row d
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int pa = p0 + 2 * e, pb = pa + 1;
            const int ka = (pa / 16) * 16 + acc_key(pa % 16), kb = (pb / 16) * 16 + acc_key(pb % 16);
            w[e] = uint32_t(sV[ka * KST + d]) | (uint32_t(sV[kb * KST + d]) << 16);
        }
        *reinterpret_cast<u32x4*>(vt + d * BK + p0) = u32x4{w[0], w[1], w[2], w[3]};
    }
}

__global__ __launch_bounds__(256, 2) void attn_prefill_kernel(
    const uint16_t* __restrict__ Q, int Tq, int Hq, int hkv, const int64_t* __restrict__ mem_off, int64_t cap,
    int64_t max_rows, int L, int q_offset, float qscale, const float2* __restrict__ rope, int max_pos,
    int64_t KP, const uint16_t* __restrict__ Kc, const uint16_t* __restrict__ Vt, uint16_t* __restrict__ O) {
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
    const int64_t bg = b * hkv + g;

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
    int64_t r0, M;
    mem_range(mem_off, b, cap, max_rows, r0, M);
    const int last_q = (i0 + BQ < Tq ? i0 + BQ : Tq) - 1;
    const int64_t jmax = int64_t(L - Tq) + last_q;                 // last local key any token here sees
    const int n_tiles = int((M + jmax + 1 + BK - 1) / BK);
    const int qi = i0 + wave * 32 + lane % 32;                      // this lane's query token
    const int64_t lim = int64_t(L - Tq) + qi;                       // local key j visible iff j <= lim
    const int q_lo = i0 + wave * 32;                                // the wave's first token
    const int q_hi = (q_lo + 31 < Tq ? q_lo + 31 : Tq - 1);         // and last valid one
    const bool wave_live = q_lo < Tq;
    const bool wave_whole = q_lo + 31 < Tq;
    const int64_t lim_lo = int64_t(L - Tq) + q_lo, lim_hi = int64_t(L - Tq) + q_hi;

    float m_run = -INFINITY, l_run = 0.f;
    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;

    // ---- register prefetch of one 64-key tile of Kc and Vt (16 KB each, contiguous)
    const uint16_t* kc = Kc + bg * KP * DH;
    const uint16_t* vtb = Vt + bg * KP * DH;
    u32x4 rk[4], rv[4];
    auto fetch = [&](int t) {
        const u32x4* ks = reinterpret_cast<const u32x4*>(kc + int64_t(t) * BK * DH);
        const u32x4* vs = reinterpret_cast<const u32x4*>(vtb + int64_t(t) * BK * DH);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            rk[j] = ks[tid + 256 * j];
            rv[j] = vs[tid + 256 * j];
        }
    };
    if (n_tiles > 0) fetch(0);

    for (int t = 0; t < n_tiles; ++t) {
        const int64_t k0 = int64_t(t) * BK;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int u = tid + 256 * j;
            *reinterpret_cast<u32x4*>(sK + (u / 16) * KST + (u % 16) * 8) = rk[j];
            *reinterpret_cast<u32x4*>(sVt + (u / 8) * VST + (u % 8) * 8) = rv[j];
        }
        __syncthreads();
        if (t + 1 < n_tiles) fetch(t + 1);

        // tile class for this wave: every key visible to every token / none to any
        const int64_t k_last = k0 + BK - 1;
        const bool all_vis = wave_whole && (k_last < M || (k_last - M) <= lim_lo);
        const bool none_vis = !wave_live || (k0 >= M && (k0 - M) > lim_hi);
        if (!none_vis) {
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
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + (tt * 32 + lane % 32) * KST + ks * 16 +
                                                                      (lane / 32) * 8);
                    s[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[tt], 0, 0, 0);
                }

            // ---- mask (edge tiles only) and tile max; lanes l and l+32 share a query
            if (!all_vis) {
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int64_t key = k0 + tt * 32 + (i / 4) * 8 + (lane / 32) * 4 + (i % 4);
                        const bool vis = (key < M || (key - M) <= lim) && qi < Tq;
                        s[tt][i] = vis ? s[tt][i] : -INFINITY;
                    }
            }
            float mt = -INFINITY;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[tt][i]);
            mt = fmaxf(mt, __shfl_xor(mt, 32));

            // ---- lazy running max: raise it only past m + kLazy
            const bool raise = mt > m_run + kLazy;
            if (__any(raise)) {
                const float m_new = raise ? mt : m_run;
                const float corr = raise ? (m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new)) : 1.f;
                l_run *= corr;
                m_run = m_new;
                // register i holds query (i/4)*8 + (lane/32)*4 + i%4 of this wave
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float f = __shfl(corr, (i / 4) * 8 + (lane / 32) * 4 + (i % 4));
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) o[dt][i] *= f;
                }
            }
            float rs = 0.f;
            if (all_vis) {
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const float p = __builtin_amdgcn_exp2f(s[tt][i] - m_run);
                        s[tt][i] = p;
                        rs += p;
                    }
            } else {
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const float p = (s[tt][i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[tt][i] - m_run);
                        s[tt][i] = p;
                        rs += p;
                    }
            }
            rs += __shfl_xor(rs, 32);
            l_run += rs;

            // ---- O += P . V over 4 k-steps of 16 keys, in accumulator order; operands
            // are assembled as packed dwords and bit-cast whole
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int tt = ks / 2, sp = ks % 2;
                const u32x4 pw = {pack_bf16x2(s[tt][sp * 8 + 0], s[tt][sp * 8 + 1]),
                                  pack_bf16x2(s[tt][sp * 8 + 2], s[tt][sp * 8 + 3]),
                                  pack_bf16x2(s[tt][sp * 8 + 4], s[tt][sp * 8 + 5]),
                                  pack_bf16x2(s[tt][sp * 8 + 6], s[tt][sp * 8 + 7])};
                const bf16x8 pa = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const bf16x8 vb = *reinterpret_cast<const bf16x8*>(sVt + (dt * 32 + lane % 32) * VST + ks * 16 +
                                                                       (lane / 32) * 8);
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, vb, o[dt], 0, 0, 0);
                }
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

int64_t keys_padded(int64_t max_rows, int L) { return ceil_div(max_rows + L, int64_t(BK)) * BK; }

}  // namespace

bool attn_mfma_applicable(const AttnArgs& a) {
    return a.dt == MSA_BF16 && a.D == DH && a.Tq >= 64;
}

size_t attn_mfma_workspace(msa_dtype dt, int64_t B, int Tq, int Hq, int Hkv, int D, int64_t max_rows, int L) {
    (void)Hq;
    if (dt != MSA_BF16 || D != DH || Tq < 64) return 0;
    const size_t one = size_t(B) * Hkv * keys_padded(max_rows, L) * DH * 2;
    return 2 * align256(one);
}

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t st) {
    const int64_t KP = keys_padded(a.max_rows, a.L);
    const size_t one = size_t(a.B) * a.Hkv * KP * DH * 2;
    uint16_t* Kc = static_cast<uint16_t*>(a.ws);
    uint16_t* Vt = reinterpret_cast<uint16_t*>(static_cast<char*>(a.ws) + align256(one));
    hipLaunchKernelGGL(attn_pack_kernel, dim3(unsigned(KP / BK), unsigned(a.Hkv), unsigned(a.B)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(a.KVmem), a.mem_off, a.mem_rows_cap, a.max_rows,
                       static_cast<const uint16_t*>(a.K_local), static_cast<const uint16_t*>(a.V_local), a.L, a.Hkv,
                       a.q_offset, a.rope_cs, a.max_pos, KP, Kc, Vt);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const dim3 grid(unsigned(ceil_div(a.Tq, BQ)), unsigned(a.Hq), unsigned(a.B));
    hipLaunchKernelGGL(attn_prefill_kernel, grid, dim3(256), 0, st, static_cast<const uint16_t*>(a.Q), a.Tq, a.Hq,
                       a.Hkv, a.mem_off, a.mem_rows_cap, a.max_rows, a.L, a.q_offset, a.scale * kLog2e, a.rope_cs,
                       a.max_pos, KP, Kc, Vt, static_cast<uint16_t*>(a.O));
    return hipGetLastError();
}

}  // namespace msa
