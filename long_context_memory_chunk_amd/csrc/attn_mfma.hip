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
// attn_pack_kernel builds, once per (query b, KV head g), the key space as the
// matrix cores read it, in the workspace, one 16 KB block per 64-key tile:
//   Kc  keys: the M_b memory rows as stored, then the L local keys rotated at
//       q_offset + j (fp32, rounded once to bf16), then zeros up to KP (a
//       multiple of 64); row r of a tile holds its 16 16-byte units with unit
//       u at position u ^ (r & 15);
//   Vt  values transposed per tile (row = dimension, 64 keys), each 16-key
//       group in the order the score accumulator holds its keys (see below);
//       row d holds its 8 units with unit u at position u ^ ((d >> 1) & 7).
// The XOR swizzles make every matrix-core operand read below hit 64 distinct
// LDS banks per 16 lanes, and a tile is copied to LDS as one contiguous block.
// Every head of the group and every query tile reads these instead of
// rotating and transposing the same keys again.
//
// attn_prefill_kernel: a workgroup (8 waves) owns 256 query tokens of one query
// head h (KV head h / G); wave w owns tokens 32w .. 32w+31 and keeps them,
// rotated and scaled, as matrix-core operands in registers.  Keys come 64 at a
// time, up to the last local key the workgroup can see, through a ring of four
// LDS tile slots filled by direct global->LDS copies three tiles ahead.
// Iteration t of the key loop does, per wave:
//   * the tile max of S(t) and, rarely, a raise of the running max;
//   * S(t+1)^T = K(t+1) . Q^T on v_mfma_f32_32x32x16_bf16 (two 32-key halves,
//     8 k-steps over d), each lane holding 32 scores of one query token
//     (lanes l and l + 32 share a token), while the vector units exponentiate,
//     sum and pack S(t): the two are independent, so they overlap;
//   * O += P(t) . V(t): the 16 keys of a k-step are contracted in the order
//     the score accumulator holds them (lane half u holds keys
//     {4u..4u+3, 8+4u..8+4u+3}), which is the order Vt stores them in, so P
//     needs no shuffle.
// The softmax runs in the log2 domain (scale 1/sqrt(d) and log2(e) folded into
// Q before its bf16 rounding); the running max m is raised only when a score
// exceeds it by more than 2^8, and l and O always use the same m, so the
// result is the same softmax.  Masks are applied only on tiles that cross a
// wave's causal edge; tiles past it are skipped by that wave.  Workgroups take
// the heaviest query tiles first, and when the (query, head) count is a
// multiple of the 8 XCDs, consecutive heads (one KV group) share an XCD and
// its L2.
#include "attn_mfma.hpp"
#include "lds_dma.hpp"

namespace msa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64, DH = 128;
constexpr int kWaves = 8;                  // waves per workgroup
constexpr int BQ = kWaves * 32;            // query tokens per workgroup
constexpr int kTileUnits = BK * DH / 8;    // 16-byte units of one K (or V) tile: 1024 (16 KB)
constexpr int kStages = 4;                 // LDS ring: three tiles in flight behind the one in use
constexpr int kXcds = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.f;               // raise the running max only past m + 8 (a factor 2^8)

// Position in a 16-key group -> key in that group (the score accumulator's order).
__device__ __forceinline__ int acc_key(int p) {
    const int u = p / 8, e = p % 8;
    return (e / 4) * 8 + 4 * u + (e % 4);
}

// Unit positions inside a tile (16-byte units).
__host__ __device__ inline int k_unit(int row, int u) { return row * 16 + (u ^ (row & 15)); }
__host__ __device__ inline int v_unit(int d, int u) { return d * 8 + (u ^ ((d >> 1) & 7)); }

constexpr int KST = DH + 8;      // V staging row stride in LDS (bf16), pack kernel only

__global__ __launch_bounds__(256) void attn_pack_kernel(
    const uint16_t* __restrict__ KVmem, const int64_t* __restrict__ mem_off, int64_t cap, int64_t max_rows,
    const uint16_t* __restrict__ Kl, const uint16_t* __restrict__ Vl, int L, int hkv, int q_offset,
    const float2* __restrict__ rope, int max_pos, int64_t KP, u32x4* __restrict__ Kc, u32x4* __restrict__ Vt) {
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
    u32x4* kt = Kc + (bg * (KP / BK) + tile) * kTileUnits;
    u32x4* vt = Vt + (bg * (KP / BK) + tile) * kTileUnits;

    // keys: 64 keys x 8 unit pairs (dimensions i, i + 64)
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
        kt[k_unit(kk, c / 8)] = w1;
        kt[k_unit(kk, c / 8 + 8)] = w2;
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
    for (int u = tid; u < DH * 8; u += 256) {
        const int d = u / 8, p0 = (u % 8) * 8;            // positions p0 .. p0+7 of row d
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int pa = p0 + 2 * e, pb = pa + 1;
            const int ka = (pa / 16) * 16 + acc_key(pa % 16), kb = (pb / 16) * 16 + acc_key(pb % 16);
            w[e] = uint32_t(sV[ka * KST + d]) | (uint32_t(sV[kb * KST + d]) << 16);
        }
        vt[v_unit(d, p0 / 8)] = u32x4{w[0], w[1], w[2], w[3]};
    }
}

__global__ __launch_bounds__(kWaves * 64, 1) void attn_prefill_kernel(
    const uint16_t* __restrict__ Q, int Tq, int Hq, int hkv, const int64_t* __restrict__ mem_off, int64_t cap,
    int64_t max_rows, int L, int q_offset, float qscale, const float2* __restrict__ rope, int max_pos,
    int64_t KP, const u32x4* __restrict__ Kc, const u32x4* __restrict__ Vt, uint16_t* __restrict__ O, int n_qt,
    int64_t B, float* __restrict__ lse) {
    __shared__ __attribute__((aligned(16))) u32x4 sK[kStages * kTileUnits];
    __shared__ __attribute__((aligned(16))) u32x4 sV[kStages * kTileUnits];

    // ---- which (query tile, batch, head): heaviest tiles first, one KV group per XCD
    const int64_t n_bh = B * Hq;
    const int64_t lin = blockIdx.x;
    const int rank = int(lin / n_bh);
    int64_t r = lin % n_bh;
    if (n_bh % kXcds == 0) r = (r % kXcds) * (n_bh / kXcds) + r / kXcds;
    const int qt = n_qt - 1 - rank;
    const int64_t b = r / Hq;
    const int h = int(r % Hq);

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave, half = lane / 32;
    const int G = Hq / hkv, g = h / G;
    const int64_t bg = b * hkv + g;
    const int i0 = qt * BQ;
    const int q_lo = i0 + wave * 32;                 // the wave's first token
    const int qi = q_lo + lane % 32;                 // this lane's token (a column of S^T)
    const bool q_valid = qi < Tq;

    // ---- rotated, scaled query token as B operands: qf[ks] holds d = 16 ks + 8 half + e
    bf16x8 qf[8];
    {
        const int qs = q_valid ? qi : 0;
        int pos = q_offset + (L - Tq) + qs;
        pos = pos < max_pos ? pos : max_pos - 1;
        const uint16_t* qrow = Q + ((b * Tq + qs) * Hq + h) * DH;
        const float2* cs = rope + int64_t(pos) * (DH / 2);
        const float sc = q_valid ? qscale : 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int c0 = 16 * ks + 8 * half;           // dimensions c0 .. c0+7 pair with c0+64 ..
            const u32x4 x1 = *reinterpret_cast<const u32x4*>(qrow + c0);
            const u32x4 x2 = *reinterpret_cast<const u32x4*>(qrow + c0 + DH / 2);
            float y1[8], y2[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float a = (e & 1) ? bf16_hi(x1[e / 2]) : bf16_lo(x1[e / 2]);
                const float bb = (e & 1) ? bf16_hi(x2[e / 2]) : bf16_lo(x2[e / 2]);
                const float2 rc = cs[c0 + e];
                y1[e] = (a * rc.x - bb * rc.y) * sc;
                y2[e] = (bb * rc.x + a * rc.y) * sc;
            }
            qf[ks] = __builtin_bit_cast(bf16x8, (u32x4{pack_bf16x2(y1[0], y1[1]), pack_bf16x2(y1[2], y1[3]),
                                                       pack_bf16x2(y1[4], y1[5]), pack_bf16x2(y1[6], y1[7])}));
            qf[ks + 4] = __builtin_bit_cast(bf16x8, (u32x4{pack_bf16x2(y2[0], y2[1]), pack_bf16x2(y2[2], y2[3]),
                                                           pack_bf16x2(y2[4], y2[5]), pack_bf16x2(y2[6], y2[7])}));
        }
    }

    // ---- key space of this workgroup and of this wave
    int64_t r0, M;
    mem_range(mem_off, b, cap, max_rows, r0, M);
    const int last_q = (i0 + BQ < Tq ? i0 + BQ : Tq) - 1;
    const int n_tiles = int((M + int64_t(L - Tq) + last_q + 1 + BK - 1) / BK);
    const int q_hi = (q_lo + 31 < Tq ? q_lo + 31 : Tq - 1);
    const bool wave_live = q_lo < Tq;
    const bool wave_whole = q_lo + 31 < Tq;
    const int64_t lim_lo = int64_t(L - Tq) + q_lo;   // local key j visible to every token of the wave iff j <= lim_lo
    const int wave_tiles = wave_live ? int((M + int64_t(L - Tq) + q_hi + 1 + BK - 1) / BK) : 0;
    // key index (in the tile's key space) up to which this lane's token sees
    const int64_t see = q_valid ? M + int64_t(L - Tq) + qi : -1;

    // ---- direct copies of tile t into ring slot t % kStages: 8 waves x 2 x 1 KB per tensor
    const u32x4* kg = Kc + bg * (KP / BK) * kTileUnits;
    const u32x4* vg = Vt + bg * (KP / BK) * kTileUnits;
    const uint32_t ldsK = lds_addr(sK), ldsV = lds_addr(sV);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t voff = uint32_t(lane) * 16u;
    auto dma = [&](int t) {
        const uint32_t slot = uint32_t(t % kStages) * kTileUnits;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int piece = (i * kWaves + wave_u) * kWave;
            lds_copy16_s(kg + int64_t(t) * kTileUnits + piece, voff, ldsK + (slot + piece) * 16);
            lds_copy16_s(vg + int64_t(t) * kTileUnits + piece, voff, ldsV + (slot + piece) * 16);
        }
    };
    constexpr int kCopies = 4;                       // copies per wave per tile

    // S(t)^T for this wave: rows = the tile's keys, columns = the wave's tokens
    auto scores = [&](int t, f32x16 (&s)[2]) {
        const u32x4* kt = sK + (t % kStages) * kTileUnits;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[tt][i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, kt[k_unit(tt * 32 + lane % 32, 2 * ks + half)]);
                s[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[tt], 0, 0, 0);
            }
    };

    float m_run = -INFINITY, l_run = 0.f;
    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;

    // tile max of S(t) (masked on edge tiles) and the lazy raise of the running max
    auto tile_max = [&](f32x16 (&s)[2], int t, bool full) {
        if (!full) {
            int64_t thr64 = see - int64_t(t) * BK;       // key offsets <= thr are visible
            thr64 = thr64 < -1 ? -1 : (thr64 > BK ? BK : thr64);
            const int thr = int(thr64);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int off = tt * 32 + (i / 4) * 8 + half * 4 + (i % 4);
                    s[tt][i] = (off <= thr) ? s[tt][i] : -INFINITY;
                }
        }
        float mt = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[tt][i]);
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const bool raise = mt > m_run + kLazy;
        if (__any(raise)) {
            const float m_new = raise ? mt : m_run;
            const float corr = raise ? (m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new)) : 1.f;
            l_run *= corr;
            m_run = m_new;
            // register i of O holds token (i/4)*8 + half*4 + i%4 of this wave
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float f = __shfl(corr, (i / 4) * 8 + half * 4 + (i % 4));
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) o[dt][i] *= f;
            }
        }
    };
    // P(t) = exp2(S - m) packed as A operands of the 4 k-steps; row sums into l.
    // On edge tiles a masked score gives 0 even where m is still -inf (a token
    // past Tq, which sees nothing).
    auto probs = [&](const f32x16 (&s)[2], bf16x8 (&pa)[4], bool full) {
        float rs = 0.f;
        float p[2][16];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float e = __builtin_amdgcn_exp2f(s[tt][i] - m_run);
                p[tt][i] = (full || s[tt][i] != -INFINITY) ? e : 0.f;
                rs += p[tt][i];
            }
        rs += __shfl_xor(rs, 32);
        l_run += rs;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int tt = ks / 2, sp = (ks % 2) * 8;
            pa[ks] = __builtin_bit_cast(bf16x8, (u32x4{pack_bf16x2(p[tt][sp + 0], p[tt][sp + 1]),
                                                       pack_bf16x2(p[tt][sp + 2], p[tt][sp + 3]),
                                                       pack_bf16x2(p[tt][sp + 4], p[tt][sp + 5]),
                                                       pack_bf16x2(p[tt][sp + 6], p[tt][sp + 7])}));
        }
    };
    auto pv = [&](int t, const bf16x8 (&pa)[4]) {
        const u32x4* vt = sV + (t % kStages) * kTileUnits;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const bf16x8 vb = __builtin_bit_cast(bf16x8, vt[v_unit(dt * 32 + lane % 32, 2 * ks + half)]);
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[ks], vb, o[dt], 0, 0, 0);
            }
    };
    // every key of tile t visible to every token of the wave
    auto tile_full = [&](int t) { return wave_whole && int64_t(t) * BK + BK - 1 <= M + lim_lo; };

    // ---- prologue: three tiles in flight, S(0)
    for (int t = 0; t < kStages - 1 && t < n_tiles; ++t) dma(t);
    if (n_tiles >= 3) MSA_WAIT_VMCNT(2 * kCopies);
    else if (n_tiles == 2) MSA_WAIT_VMCNT(kCopies);
    else MSA_WAIT_VMCNT(0);
    __syncthreads();
    f32x16 s_cur[2];
    if (wave_tiles > 0) scores(0, s_cur);

    for (int t = 0; t < n_tiles; ++t) {
        // tile t+1 in LDS for every wave, and every wave done with the slot tile t+3 reuses
        if (t + 2 < n_tiles) MSA_WAIT_VMCNT(kCopies);
        else MSA_WAIT_VMCNT(0);
        __syncthreads();
        if (t + kStages - 1 < n_tiles) dma(t + kStages - 1);

        f32x16 s_nxt[2];
        bf16x8 pa[4];
        if (t + 1 < wave_tiles && tile_full(t)) {
            // common case: S(t+1) on the matrix cores while the vector units finish S(t)
            tile_max(s_cur, t, true);
            scores(t + 1, s_nxt);
            probs(s_cur, pa, true);
            pv(t, pa);
        } else {
            const bool full = tile_full(t);
            if (t < wave_tiles) tile_max(s_cur, t, full);
            if (t + 1 < wave_tiles) scores(t + 1, s_nxt);
            if (t < wave_tiles) {
                probs(s_cur, pa, full);
                pv(t, pa);
            }
        }
        if (t + 1 < wave_tiles) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) s_cur[tt] = s_nxt[tt];
        }
    }

    // ---- normalise and store (and the row's log-sum-exp, natural log, if asked)
    if (lse != nullptr && half == 0 && q_valid)
        lse[(b * Tq + qi) * Hq + h] = (m_run + log2f(l_run)) * kLn2;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int qr = (i / 4) * 8 + half * 4 + (i % 4);
        const float lsum = __shfl(l_run, qr);
        const int qtok = q_lo + qr;
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
    u32x4* Kc = static_cast<u32x4*>(a.ws);
    u32x4* Vt = reinterpret_cast<u32x4*>(static_cast<char*>(a.ws) + align256(one));
    hipLaunchKernelGGL(attn_pack_kernel, dim3(unsigned(KP / BK), unsigned(a.Hkv), unsigned(a.B)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(a.KVmem), a.mem_off, a.mem_rows_cap, a.max_rows,
                       static_cast<const uint16_t*>(a.K_local), static_cast<const uint16_t*>(a.V_local), a.L, a.Hkv,
                       a.q_offset, a.rope_cs, a.max_pos, KP, Kc, Vt);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int n_qt = int(ceil_div(a.Tq, BQ));
    const int64_t blocks = int64_t(n_qt) * a.B * a.Hq;
    hipLaunchKernelGGL(attn_prefill_kernel, dim3(unsigned(blocks)), dim3(kWaves * 64), 0, st,
                       static_cast<const uint16_t*>(a.Q), a.Tq, a.Hq, a.Hkv, a.mem_off, a.mem_rows_cap, a.max_rows,
                       a.L, a.q_offset, a.scale * kLog2e, a.rope_cs, a.max_pos, KP,
                       static_cast<const u32x4*>(Kc), static_cast<const u32x4*>(Vt), static_cast<uint16_t*>(a.O),
                       n_qt, a.B, a.lse);
    return hipGetLastError();
}

}  // namespace msa
