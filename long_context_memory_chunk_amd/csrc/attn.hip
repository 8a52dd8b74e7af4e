// Stage 3: GQA attention over [selected K̄/V̄ ; local K/V] with global RoPE.
//
// Source: news.neo-ai.one MSA article, 全体設計 › アーキテクチャ (Fig. 2): the
// compressed K/V of the selected documents are concatenated with the query's
// local K/V for autoregressive decoding, and global RoPE shifts the query's
// start index by k so the order is background -> query -> generation;
// 推論パイプライン (Fig. 3), third stage (sparse generation).
//
// Key space of query (b, i): first the M_b memory rows of query b (visible to
// every query token, used as stored), then the local keys j = 0 ..
// (L - Tq) + i (causal), rotated here at position q_offset + j.  The query is
// rotated at q_offset + (L - Tq) + i.
//
// Three kernels compute it; launch_attn takes the first that applies:
//   attn_prefill_kernel (attn_mfma.hip)  bf16, d = 128, long query blocks:
//                                        matrix cores.
//   attn_decode_kernel (below)           bf16, d = 128, G in {1, 2, 4}:
//                                        decode and short queries, laid out
//                                        for HBM bandwidth.
//   attn_split_kernel                    any dtype, d in {64, 128}, any G.
// The last two write partial (m, l, o) per key split; attn_combine merges
// them exactly.  Every path can also write each row's log-sum-exp (the
// statistic the backward in attn_bwd.hip recomputes the softmax from).
//
// attn_split (vector ALU, any Tq): a workgroup owns one (b, i, kv head g) and
// the G = Hq/Hkv query heads that read g, so every key row loaded is used G
// times.  Keys are taken 256 at a time: one key per thread for the logits,
// then for P.V each wave walks 64 of the keys, loading each V row as one
// coalesced wave access (D/64 elements per lane) and accumulating all G
// heads in registers; an online softmax runs across the 256-key splits the
// workgroup owns, and the four waves' partial sums meet in LDS at the end.
// Splits are dealt to P workgroups.
#include "common.hpp"
#include "launch.hpp"
#include "attn_mfma.hpp"

namespace msa {
namespace {

constexpr int kSplit = 256;

// DPL consecutive elements of one row as floats (DPL = D / 64 per lane).
template <typename T, int DPL> struct LanePart;
template <> struct LanePart<bf16_t, 2> {
    __device__ __forceinline__ static void load(const bf16_t* p, float* v) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
        v[0] = bf16_lo(w); v[1] = bf16_hi(w);
    }
};
template <> struct LanePart<bf16_t, 1> {
    __device__ __forceinline__ static void load(const bf16_t* p, float* v) { v[0] = bf16_to_f32(p->bits); }
};
template <> struct LanePart<float, 2> {
    __device__ __forceinline__ static void load(const float* p, float* v) {
        const float2 w = *reinterpret_cast<const float2*>(p);
        v[0] = w.x; v[1] = w.y;
    }
};
template <> struct LanePart<float, 1> {
    __device__ __forceinline__ static void load(const float* p, float* v) { v[0] = *p; }
};

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void attn_split_kernel(
    const T* __restrict__ Q, int Tq, int Hq, int hkv, const T* __restrict__ KVmem,
    const int64_t* __restrict__ mem_off, int64_t cap, int64_t max_rows,
    const T* __restrict__ Kl, const T* __restrict__ Vl, int L, int q_offset, float scale,
    const float2* __restrict__ rope_cs, int max_pos, int P,
    float* __restrict__ part_o, float2* __restrict__ part_ml) {
    constexpr int VEC = Vec16<T>::kN;
    constexpr int HALF = D / 2;
    constexpr int DPL = D / kWave;
    __shared__ float qs[G][D];
    __shared__ float lg[G][kSplit];
    __shared__ float s_corr[G];
    __shared__ float s_m[G];
    __shared__ float s_l[G];
    __shared__ float red[4][G][D];

    const int tid = threadIdx.x;
    const int lane = tid % kWave, wave = tid / kWave;
    const int p = blockIdx.x;
    const int g = blockIdx.y;
    const int64_t bt = blockIdx.z;
    const int64_t b = bt / Tq;
    const int i = int(bt % Tq);

    // rotate and scale the G query heads of this group
    int pos_q = q_offset + (L - Tq) + i;
    pos_q = pos_q < max_pos ? pos_q : max_pos - 1;
    for (int idx = tid; idx < G * HALF; idx += 256) {
        const int hh = idx / HALF, ii = idx % HALF;
        const int64_t qb = ((bt * Hq) + g * G + hh) * D;
        const float x1 = Elem<T>::load(Q, qb + ii), x2 = Elem<T>::load(Q, qb + ii + HALF);
        const float2 cs = rope_cs[int64_t(pos_q) * HALF + ii];
        qs[hh][ii] = (x1 * cs.x - x2 * cs.y) * scale;
        qs[hh][ii + HALF] = (x2 * cs.x + x1 * cs.y) * scale;
    }
    if (tid < G) { s_m[tid] = -INFINITY; s_l[tid] = 0.f; }

    int64_t r0 = mem_off[b], r1 = mem_off[b + 1];
    r0 = r0 < 0 ? 0 : (r0 > cap ? cap : r0);
    r1 = r1 < r0 ? r0 : (r1 > cap ? cap : r1);
    if (r1 - r0 > max_rows) r1 = r0 + max_rows;
    const int64_t M = r1 - r0;
    const int64_t n_vis = int64_t(L - Tq) + i + 1;
    const int64_t total = M + n_vis;
    const int64_t n_splits = (total + kSplit - 1) / kSplit;
    const int64_t row_elems = int64_t(hkv) * D;

    // P.V accumulators of this wave: its 64-key share of every split, DPL dims per lane
    float o[G][DPL];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[hh][e] = 0.f;
    __syncthreads();

    for (int64_t sp = p; sp < n_splits; sp += P) {
        // ---- logits: one key per thread
        const int64_t kk = sp * kSplit + tid;
        float acc[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) acc[hh] = 0.f;
        if (kk < total) {
            if (kk < M) {
                const T* kr = KVmem + (r0 + kk) * 2 * row_elems + int64_t(g) * D;
#pragma unroll
                for (int i0 = 0; i0 < D; i0 += VEC) {
                    float x[VEC];
                    Vec16<T>::load(kr + i0, x);
#pragma unroll
                    for (int hh = 0; hh < G; ++hh) {
                        float a = acc[hh];
#pragma unroll
                        for (int u = 0; u < VEC; ++u) a += x[u] * qs[hh][i0 + u];
                        acc[hh] = a;
                    }
                }
            } else {
                const int64_t j = kk - M;
                const T* kr = Kl + ((b * L + j) * hkv + g) * D;
                int pos = q_offset + int(j);
                pos = pos < max_pos ? pos : max_pos - 1;
                const float2* cs = rope_cs + int64_t(pos) * HALF;
#pragma unroll
                for (int i0 = 0; i0 < HALF; i0 += VEC) {
                    float x1[VEC], x2[VEC], y1[VEC], y2[VEC];
                    Vec16<T>::load(kr + i0, x1);
                    Vec16<T>::load(kr + i0 + HALF, x2);
#pragma unroll
                    for (int u = 0; u < VEC; ++u) {
                        const float2 c = cs[i0 + u];
                        y1[u] = x1[u] * c.x - x2[u] * c.y;
                        y2[u] = x2[u] * c.x + x1[u] * c.y;
                    }
#pragma unroll
                    for (int hh = 0; hh < G; ++hh) {
                        float a = acc[hh];
#pragma unroll
                        for (int u = 0; u < VEC; ++u)
                            a += y1[u] * qs[hh][i0 + u] + y2[u] * qs[hh][i0 + HALF + u];
                        acc[hh] = a;
                    }
                }
            }
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) lg[hh][tid] = (kk < total) ? acc[hh] : -INFINITY;
        __syncthreads();

        // ---- softmax bookkeeping per head (wave w owns heads w, w+4, ...)
        for (int hh = wave; hh < G; hh += 4) {
            float mx = -INFINITY;
            for (int t = lane; t < kSplit; t += kWave) mx = fmaxf(mx, lg[hh][t]);
            mx = wave_max(mx);
            const float m_old = s_m[hh];
            const float m_new = fmaxf(m_old, mx);
            float sum = 0.f;
            for (int t = lane; t < kSplit; t += kWave) {
                const float e = (lg[hh][t] == -INFINITY) ? 0.f : expf(lg[hh][t] - m_new);
                lg[hh][t] = e;
                sum += e;
            }
            sum = wave_sum(sum);
            if (lane == 0) {
                const float corr = (m_old == -INFINITY) ? 0.f : expf(m_old - m_new);
                s_corr[hh] = corr;
                s_l[hh] = s_l[hh] * corr + sum;
                s_m[hh] = m_new;
            }
        }
        __syncthreads();

        // ---- P.V: wave w takes keys w*64 .. w*64+63 of the split, one V row per step
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const float c = s_corr[hh];
#pragma unroll
            for (int e = 0; e < DPL; ++e) o[hh][e] *= c;
        }
        const int64_t k_begin = sp * kSplit + wave * kWave;
        int nk = int((total - k_begin) < kWave ? (total - k_begin) : kWave);
        nk = nk < 0 ? 0 : nk;
#pragma unroll 4
        for (int t = 0; t < nk; ++t) {
            const int64_t key = k_begin + t;
            const T* vr = (key < M) ? KVmem + (r0 + key) * 2 * row_elems + row_elems + int64_t(g) * D
                                    : Vl + ((b * L + (key - M)) * hkv + g) * D;
            float v[DPL];
            LanePart<T, DPL>::load(vr + lane * DPL, v);
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                const float pw = lg[hh][wave * kWave + t];
#pragma unroll
                for (int e = 0; e < DPL; ++e) o[hh][e] += pw * v[e];
            }
        }
        __syncthreads();
    }

    // ---- sum the four waves' partial P.V and write this workgroup's partial
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < DPL; ++e) red[wave][hh][lane * DPL + e] = o[hh][e];
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += 256) {
        const int hh = idx / D, dd = idx % D;
        const float v = (red[0][hh][dd] + red[1][hh][dd]) + (red[2][hh][dd] + red[3][hh][dd]);
        part_o[((bt * Hq + g * G + hh) * P + p) * D + dd] = v;
    }
    if (tid < G) part_ml[(bt * Hq + g * G + tid) * P + p] = make_float2(s_m[tid], s_l[tid]);
}

// ---------------------------------------------------------------- bf16, d = 128
//
// attn_decode_kernel: the same key space and mask as attn_split_kernel, laid
// out for HBM bandwidth.  A workgroup (4 waves) owns NC consecutive 64-key
// chunks of one (b, i, kv head g) and the G query heads that read g; wave w
// takes keys 16w .. 16w+15 of every chunk.  16 lanes hold one key: lane c of
// the 16 owns bytes 16c .. 16c+15 of the 256-byte row, so one wave instruction
// reads four whole rows; a lane's keys in a chunk are its key slot s = lane /
// 16 plus 4 it, it = 0 .. 3.  The next chunk's K rows are loaded while this
// chunk is used (two register buffers), and its V rows as soon as this
// chunk's P.V is done.  A local key's RoPE pair
// (i, i + 64) sits in lanes c and c + 8 of the same row of 16 lanes and is
// exchanged with DPP row_ror:8; a lane's local keys in a chunk are 4 positions
// apart, so its cos/sin advance by the fixed rotation of 4 positions (angle
// addition) from the table value at its first local key of the chunk.  The G
// dot products are summed over the 16 lanes with DPP.  Each wave keeps an
// online softmax in registers (log2 domain, scale and log2(e) folded into the
// query; the running max is raised only past m + 2^8 = kLazy); the slots and
// the waves are merged once, at the end, into one partial (m, l, o) per
// workgroup, which attn_combine_kernel merges with the others.

__device__ __forceinline__ uint32_t ror8_16(uint32_t v) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x128, 0xF, 0xF, false));   // row_ror:8
}

constexpr int kDecodeChunk = 64;             // keys per chunk
constexpr float kDecodeLazy = 8.f;           // log2 units: raise the running max only past m + 8
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;

template <int G>
__global__ __launch_bounds__(256, 2) void attn_decode_kernel(
    const bf16_t* __restrict__ Q, int Tq, int Hq, int hkv, const bf16_t* __restrict__ KVmem,
    const int64_t* __restrict__ mem_off, int64_t cap, int64_t max_rows,
    const bf16_t* __restrict__ Kl, const bf16_t* __restrict__ Vl, int L, int q_offset, float qscale,
    const float2* __restrict__ rope_cs, int max_pos, int P, int NC,
    float* __restrict__ part_o, float2* __restrict__ part_ml) {
    constexpr int D = 128, CK = kDecodeChunk, NIT = 4;
    __shared__ float red[4][G][D];
    __shared__ float s_m[4][G], s_l[4][G];

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int slot = lane / 16, c = lane % 16;
    const float sgn = (c & 8) ? 1.f : -1.f;      // first half: x1 c - x2 s; second: x2 c + x1 s
    const int p = blockIdx.x, g = blockIdx.y;
    const int64_t bt = blockIdx.z;
    const int64_t b = bt / Tq;
    const int i = int(bt % Tq);

    int64_t r0 = mem_off[b], r1 = mem_off[b + 1];
    r0 = r0 < 0 ? 0 : (r0 > cap ? cap : r0);
    r1 = r1 < r0 ? r0 : (r1 > cap ? cap : r1);
    if (r1 - r0 > max_rows) r1 = r0 + max_rows;
    const int64_t M = r1 - r0;
    const int64_t total = M + int64_t(L - Tq) + i + 1;
    const int64_t row_elems = int64_t(hkv) * D;
    const int64_t hrow = bt * Hq + int64_t(g) * G;   // first query head row of this group
    const int64_t n_chunks = (total + CK - 1) / CK;
    const int64_t cb = int64_t(p) * NC;
    const int64_t ce = (cb + NC < n_chunks) ? cb + NC : n_chunks;

    if (cb >= ce) {                              // no keys here: an empty partial
        for (int idx = tid; idx < G * D; idx += 256) part_o[((hrow + idx / D) * P + p) * D + idx % D] = 0.f;
        if (tid < G) part_ml[(hrow + tid) * P + p] = make_float2(-INFINITY, 0.f);
        return;
    }

    // ---- this lane's 8 elements of the G rotated, scaled query heads
    float q[G][8];
    float2 step[8];
    {
        u32x4 qw[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) qw[hh] = *reinterpret_cast<const u32x4*>(Q + (hrow + hh) * D + c * 8);
        int pos_q = q_offset + (L - Tq) + i;
        pos_q = pos_q < max_pos ? pos_q : max_pos - 1;
        const float2* cs_q = rope_cs + int64_t(pos_q) * (D / 2) + (c % 8) * 8;
        const float2* st = rope_cs + int64_t(4 < max_pos ? 4 : max_pos - 1) * (D / 2) + (c % 8) * 8;
        float2 cq[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) { cq[e] = cs_q[e]; step[e] = st[e]; }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const u32x4 w = qw[hh];
            const u32x4 pw = {ror8_16(w[0]), ror8_16(w[1]), ror8_16(w[2]), ror8_16(w[3])};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = (e & 1) ? bf16_hi(w[e / 2]) : bf16_lo(w[e / 2]);
                const float px = (e & 1) ? bf16_hi(pw[e / 2]) : bf16_lo(pw[e / 2]);
                q[hh][e] = (x * cq[e].x + sgn * px * cq[e].y) * qscale;
            }
        }
    }

    // ---- chunk loads: the K rows of this lane's 4 keys (keys past the end load
    // the last valid key, in bounds, and are masked) with the cos/sin of its
    // first local key in the chunk, two buffers deep; and the V rows, one
    // buffer, loaded as soon as the previous chunk's P.V has used them
    struct Buf {
        u32x4 k[NIT];
        float2 seed[8];
    };
    u32x4 vbuf[NIT];
    auto key_ptr = [&](int64_t key, bool value) {
        key = key < total ? key : total - 1;
        return (key >= M) ? (value ? Vl : Kl) + ((b * L + (key - M)) * hkv + g) * D
                          : KVmem + (r0 + key) * 2 * row_elems + (value ? row_elems : 0) + int64_t(g) * D;
    };
    auto load_k = [&](int64_t cidx, Buf& bf) {
        const int64_t kb = cidx * CK + wave * 16 + slot;
#pragma unroll
        for (int it = 0; it < NIT; ++it)
            bf.k[it] = *reinterpret_cast<const u32x4*>(key_ptr(kb + 4 * it, false) + c * 8);
        const int64_t fl = (M > kb) ? (M - kb + 3) / 4 : 0;          // first it with key >= M
        int64_t pos = int64_t(q_offset) + kb + 4 * fl - M;
        pos = pos < 0 ? 0 : (pos < max_pos ? pos : max_pos - 1);
        const float2* cs = rope_cs + pos * (D / 2) + (c % 8) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) bf.seed[e] = cs[e];
    };
    auto load_v = [&](int64_t cidx) {
        const int64_t kb = cidx * CK + wave * 16 + slot;
#pragma unroll
        for (int it = 0; it < NIT; ++it)
            vbuf[it] = *reinterpret_cast<const u32x4*>(key_ptr(kb + 4 * it, true) + c * 8);
    };

    float m[G], l[G], o[G][8];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        m[hh] = -INFINITY;
        l[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
    }

    auto process = [&](int64_t cidx, const Buf& bf, bool next) {
        const int64_t kb = cidx * CK + wave * 16 + slot;
        const int64_t fl = (M > kb) ? (M - kb + 3) / 4 : 0;
        float2 rot[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) rot[e] = bf.seed[e];
        float lg[G][NIT];
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const bool valid = kb + 4 * it < total;
            const u32x4 w = bf.k[it];
            float y[8];
            if (it >= fl) {                      // local key: rotate
                if (it > fl) {                   // advance cos/sin by 4 positions
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float2 r = rot[e];
                        rot[e] = make_float2(r.x * step[e].x - r.y * step[e].y, r.y * step[e].x + r.x * step[e].y);
                    }
                }
                const u32x4 pw = {ror8_16(w[0]), ror8_16(w[1]), ror8_16(w[2]), ror8_16(w[3])};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = (e & 1) ? bf16_hi(w[e / 2]) : bf16_lo(w[e / 2]);
                    const float px = (e & 1) ? bf16_hi(pw[e / 2]) : bf16_lo(pw[e / 2]);
                    y[e] = x * rot[e].x + sgn * px * rot[e].y;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = (e & 1) ? bf16_hi(w[e / 2]) : bf16_lo(w[e / 2]);
            }
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) d += y[e] * q[hh][e];
                d = group_sum<16>(d);
                lg[hh][it] = valid ? d : -INFINITY;
            }
        }
        // online softmax per head over the wave's 16 keys (the max is the same in
        // every lane); the probabilities replace the logits in place
        float (&pr)[G][NIT] = lg;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            float mx = fmaxf(fmaxf(lg[hh][0], lg[hh][1]), fmaxf(lg[hh][2], lg[hh][3]));
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            if (mx > m[hh] + kDecodeLazy) {
                const float corr = (m[hh] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[hh] - mx);
                l[hh] *= corr;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[hh][e] *= corr;
                m[hh] = mx;
            }
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                pr[hh][it] = (lg[hh][it] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(lg[hh][it] - m[hh]);   // same element
                l[hh] += pr[hh][it];
            }
        }
        // P.V in the same layout
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const u32x4 w = vbuf[it];
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (e & 1) ? bf16_hi(w[e / 2]) : bf16_lo(w[e / 2]);
#pragma unroll
            for (int hh = 0; hh < G; ++hh)
#pragma unroll
                for (int e = 0; e < 8; ++e) o[hh][e] += pr[hh][it] * v[e];
        }
        if (next) load_v(cidx + 1);
    };

    // ---- chunks cb .. ce-1, the next one's loads in flight behind this one
    Buf A, Bb;
    load_k(cb, A);
    load_v(cb);
    for (int64_t cc = cb; cc < ce; cc += 2) {
        if (cc + 1 < ce) load_k(cc + 1, Bb);
        process(cc, A, cc + 1 < ce);
        if (cc + 1 >= ce) break;
        if (cc + 2 < ce) load_k(cc + 2, A);
        process(cc + 1, Bb, cc + 2 < ce);
    }

    // ---- merge the four key slots of each wave (same m), then the waves
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        l[hh] += __shfl_xor(l[hh], 16);
        l[hh] += __shfl_xor(l[hh], 32);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = o[hh][e];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            o[hh][e] = v;
        }
    }
    if (slot == 0) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[wave][hh][c * 8 + e] = o[hh][e];
    }
    if (lane == 0) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) { s_m[wave][hh] = m[hh]; s_l[wave][hh] = l[hh]; }
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += 256) {
        const int hh = idx / D, dd = idx % D;
        const float mw = fmaxf(fmaxf(s_m[0][hh], s_m[1][hh]), fmaxf(s_m[2][hh], s_m[3][hh]));
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float f = (s_m[w][hh] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s_m[w][hh] - mw);
            acc += f * red[w][hh][dd];
        }
        part_o[((hrow + hh) * P + p) * D + dd] = acc;
    }
    if (tid < G) {
        const float mw = fmaxf(fmaxf(s_m[0][tid], s_m[1][tid]), fmaxf(s_m[2][tid], s_m[3][tid]));
        float lsum = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            lsum += (s_m[w][tid] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s_m[w][tid] - mw) * s_l[w][tid];
        // the combine takes m in natural-log units
        part_ml[(hrow + tid) * P + p] = make_float2(mw == -INFINITY ? -INFINITY : mw * kLn2, lsum);
    }
}

// Merges the P partial (m, l, o) of one output row: the partials' weights
// exp(m_p - m) and the weighted row sums are computed in parallel (weights
// kept in LDS), then each thread sums its dimension over the partials with
// several loads in flight.
constexpr int kMaxParts = 1024;

template <typename T, int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(const float* __restrict__ part_o,
                                                         const float2* __restrict__ part_ml, int P,
                                                         T* __restrict__ O, float* __restrict__ lse) {
    __shared__ float s_w[kMaxParts];
    __shared__ float s_red[2][D / 64];
    const int64_t row = blockIdx.x;   // (b, i, h)
    const int dd = threadIdx.x;
    const int lane = dd % kWave, wave = dd / kWave;
    float m = -INFINITY;
    for (int p = dd; p < P; p += D) m = fmaxf(m, part_ml[row * P + p].x);
    m = wave_max(m);
    if (lane == 0) s_red[0][wave] = m;
    __syncthreads();
    m = s_red[0][0];
#pragma unroll
    for (int w = 1; w < D / 64; ++w) m = fmaxf(m, s_red[0][w]);
    float l = 0.f;
    for (int p = dd; p < P; p += D) {
        const float2 ml = part_ml[row * P + p];
        const float w = (ml.x == -INFINITY) ? 0.f : expf(ml.x - m);
        s_w[p] = w;
        l += w * ml.y;
    }
    l = wave_sum(l);
    if (lane == 0) s_red[1][wave] = l;
    __syncthreads();
    l = s_red[1][0];
#pragma unroll
    for (int w = 1; w < D / 64; ++w) l += s_red[1][w];
    float acc = 0.f;
    int p = 0;
    for (; p + 4 <= P; p += 4) {
        const float o0 = part_o[(row * P + p) * D + dd], o1 = part_o[(row * P + p + 1) * D + dd];
        const float o2 = part_o[(row * P + p + 2) * D + dd], o3 = part_o[(row * P + p + 3) * D + dd];
        acc += s_w[p] * o0;
        acc += s_w[p + 1] * o1;
        acc += s_w[p + 2] * o2;
        acc += s_w[p + 3] * o3;
    }
    for (; p < P; ++p) acc += s_w[p] * part_o[(row * P + p) * D + dd];
    Elem<T>::store(O, row * D + dd, acc / l);
    if (lse != nullptr && dd == 0) lse[row] = m + logf(l);
}

// Chunks per workgroup of attn_decode_kernel: about four workgroups per CU,
// counted from the largest key count a query may have, each taking as many
// chunks as that allows (at most 16), so its set-up and merge are spread over
// several chunks.  (Measured on the 32-query batch: 4 per CU 108.6 us, 8 per
// CU 113.9 us, 16 per CU 124.3 us; the kernel is bound by its per-key vector
// work, so more workgroups only add set-up.)
struct DecodePlan {
    int nc, P;
};

DecodePlan decode_plan(int64_t B, int Tq, int Hkv, int64_t max_rows, int L, int num_cus) {
    const int64_t chunks = ceil_div(max_rows + L, int64_t(kDecodeChunk));
    const int64_t total = B * Tq * Hkv * chunks;
    int64_t nc = total / (int64_t(num_cus) * 4);
    nc = nc < 1 ? 1 : (nc > 16 ? 16 : nc);
    if (nc > chunks) nc = chunks;
    return DecodePlan{int(nc), int(ceil_div(chunks, nc))};
}

bool decode_applicable(msa_dtype dt, int D, int Hq, int Hkv, int64_t max_rows, int L) {
    const int G = Hq / Hkv;
    return dt == MSA_BF16 && D == 128 && (G == 1 || G == 2 || G == 4) &&
           max_rows + L <= int64_t(kDecodeChunk) * kMaxParts;     // at most kMaxParts partials per row
}

int attn_parts(int64_t B, int Tq, int Hkv, int64_t max_rows, int L, int num_cus) {
    const int64_t units = B * Tq * Hkv;
    const int64_t max_splits = ceil_div(max_rows + L, kSplit);
    int64_t P = ceil_div(int64_t(2) * num_cus, units);
    if (P > max_splits) P = max_splits;
    if (P < 1) P = 1;
    return int(P);
}

template <typename T, int D, int G>
hipError_t launch_split_g(const AttnArgs& a, float* part_o, float2* part_ml, int P, hipStream_t st) {
    hipLaunchKernelGGL((attn_split_kernel<T, D, G>), dim3(unsigned(P), unsigned(a.Hkv), unsigned(a.B * a.Tq)),
                       dim3(256), 0, st, static_cast<const T*>(a.Q), a.Tq, a.Hq, a.Hkv,
                       static_cast<const T*>(a.KVmem), a.mem_off, a.mem_rows_cap, a.max_rows,
                       static_cast<const T*>(a.K_local), static_cast<const T*>(a.V_local), a.L,
                       a.q_offset, a.scale, a.rope_cs, a.max_pos, P, part_o, part_ml);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((attn_combine_kernel<T, D>), dim3(unsigned(a.B * a.Tq * a.Hq)), dim3(D), 0, st,
                       part_o, part_ml, P, static_cast<T*>(a.O), a.lse);
    return hipGetLastError();
}

template <int G>
hipError_t launch_decode_g(const AttnArgs& a, float* part_o, float2* part_ml, DecodePlan pl, hipStream_t st) {
    hipLaunchKernelGGL((attn_decode_kernel<G>), dim3(unsigned(pl.P), unsigned(a.Hkv), unsigned(a.B * a.Tq)),
                       dim3(256), 0, st, static_cast<const bf16_t*>(a.Q), a.Tq, a.Hq, a.Hkv,
                       static_cast<const bf16_t*>(a.KVmem), a.mem_off, a.mem_rows_cap, a.max_rows,
                       static_cast<const bf16_t*>(a.K_local), static_cast<const bf16_t*>(a.V_local), a.L,
                       a.q_offset, a.scale * kLog2e, a.rope_cs, a.max_pos, pl.P, pl.nc, part_o, part_ml);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((attn_combine_kernel<bf16_t, 128>), dim3(unsigned(a.B * a.Tq * a.Hq)), dim3(128), 0, st,
                       part_o, part_ml, pl.P, static_cast<bf16_t*>(a.O), a.lse);
    return hipGetLastError();
}

hipError_t launch_decode(const AttnArgs& a, float* part_o, float2* part_ml, DecodePlan pl, hipStream_t st) {
    switch (a.Hq / a.Hkv) {
        case 1: return launch_decode_g<1>(a, part_o, part_ml, pl, st);
        case 2: return launch_decode_g<2>(a, part_o, part_ml, pl, st);
        case 4: return launch_decode_g<4>(a, part_o, part_ml, pl, st);
        default: return hipErrorNotSupported;
    }
}

template <typename T, int D>
hipError_t launch_split(const AttnArgs& a, float* part_o, float2* part_ml, int P, hipStream_t st) {
    switch (a.Hq / a.Hkv) {
        case 1: return launch_split_g<T, D, 1>(a, part_o, part_ml, P, st);
        case 2: return launch_split_g<T, D, 2>(a, part_o, part_ml, P, st);
        case 4: return launch_split_g<T, D, 4>(a, part_o, part_ml, P, st);
        case 8: return launch_split_g<T, D, 8>(a, part_o, part_ml, P, st);
        case 16: return launch_split_g<T, D, 16>(a, part_o, part_ml, P, st);
        default: return hipErrorNotSupported;
    }
}

}  // namespace

bool attn_supported_group(int Hq, int Hkv) {
    const int G = Hq / Hkv;
    return G == 1 || G == 2 || G == 4 || G == 8 || G == 16;
}

size_t attn_workspace(msa_dtype dt, int64_t B, int Tq, int Hq, int Hkv, int D, int64_t max_rows,
                      int L, int num_cus) {
    const int P = decode_applicable(dt, D, Hq, Hkv, max_rows, L)
                      ? decode_plan(B, Tq, Hkv, max_rows, L, num_cus).P
                      : attn_parts(B, Tq, Hkv, max_rows, L, num_cus);
    const size_t rows = size_t(B) * Tq * Hq * P;
    size_t split = align256(rows * D * sizeof(float)) + align256(rows * sizeof(float2));
    size_t mf = attn_mfma_workspace(dt, B, Tq, Hq, Hkv, D, max_rows, L);
    return split > mf ? split : mf;
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
    if (a.B == 0 || a.Tq == 0) return hipSuccess;
    if (attn_mfma_applicable(a)) return launch_attn_mfma(a, st);
    if (decode_applicable(a.dt, a.D, a.Hq, a.Hkv, a.max_rows, a.L)) {
        const DecodePlan pl = decode_plan(a.B, a.Tq, a.Hkv, a.max_rows, a.L, a.num_cus);
        const size_t rows = size_t(a.B) * a.Tq * a.Hq * pl.P;
        float* part_o = static_cast<float*>(a.ws);
        float2* part_ml = reinterpret_cast<float2*>(static_cast<char*>(a.ws) + align256(rows * a.D * sizeof(float)));
        return launch_decode(a, part_o, part_ml, pl, st);
    }
    const int P = attn_parts(a.B, a.Tq, a.Hkv, a.max_rows, a.L, a.num_cus);
    const size_t rows = size_t(a.B) * a.Tq * a.Hq * P;
    float* part_o = static_cast<float*>(a.ws);
    float2* part_ml = reinterpret_cast<float2*>(static_cast<char*>(a.ws) + align256(rows * a.D * sizeof(float)));
    if (a.dt == MSA_BF16)
        return a.D == 128 ? launch_split<bf16_t, 128>(a, part_o, part_ml, P, st)
                          : launch_split<bf16_t, 64>(a, part_o, part_ml, P, st);
    return a.D == 128 ? launch_split<float, 128>(a, part_o, part_ml, P, st)
                      : launch_split<float, 64>(a, part_o, part_ml, P, st);
}

}  // namespace msa
