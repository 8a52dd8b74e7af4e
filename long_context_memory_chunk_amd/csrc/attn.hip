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
//   attn_decode_mfma_kernel              bf16, d = 128, G in {1, 2, 4, 8}:
//     (attn_decode_mfma.hip)             decode and short queries, scores on
//                                        the matrix cores, P . V on v_dot2.
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
#include "gather_body.hpp"

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

// Merges the P partial (m, l, o) of one output row: the partials' weights
// exp(m_p - m) and the weighted row sums are computed in parallel (weights
// kept in LDS), then each thread sums its dimension over the partials with
// several loads in flight.
constexpr int kMaxParts = 1024;

// Which of a row's P_stride partials the combine reads: all of them (mode
// 0), or, for the one-token gather + attention launch (mode 1, one query),
// the P_loc local partials and then one per rows_per memory rows actually
// gathered (mem_off[1]): the copy workgroups past the gathered rows write
// none.  (Trimming the empty partitions of the decode launch the same way,
// from mem_off, was slower: the combine then waits for mem_off before its
// first partial load.)
struct CombineTrim {
    int mode;
    const int64_t* mem_off;
    int P_loc, rows_per;
};

__device__ __forceinline__ int trim_parts(const CombineTrim& tr, int P_stride) {
    const int64_t used = tr.P_loc + (tr.mem_off[1] + tr.rows_per - 1) / tr.rows_per;
    return int(used < 1 ? 1 : (used < P_stride ? used : P_stride));
}

template <typename T, int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(const float* __restrict__ part_o,
                                                         const float2* __restrict__ part_ml, int P_stride,
                                                         T* __restrict__ O, float* __restrict__ lse,
                                                         CombineTrim tr) {
    __shared__ float s_w[kMaxParts];
    __shared__ float s_red[2][D / 64];
    const int P = tr.mode == 0 ? P_stride : trim_parts(tr, P_stride);
    const int64_t row = blockIdx.x;   // (b, i, h)
    const int dd = threadIdx.x;
    const int lane = dd % kWave, wave = dd / kWave;
    float m = -INFINITY;
    for (int p = dd; p < P; p += D) m = fmaxf(m, part_ml[row * P_stride + p].x);
    m = wave_max(m);
    if (lane == 0) s_red[0][wave] = m;
    __syncthreads();
    m = s_red[0][0];
#pragma unroll
    for (int w = 1; w < D / 64; ++w) m = fmaxf(m, s_red[0][w]);
    float l = 0.f;
    for (int p = dd; p < P; p += D) {
        const float2 ml = part_ml[row * P_stride + p];
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
        const float o0 = part_o[(row * P_stride + p) * D + dd], o1 = part_o[(row * P_stride + p + 1) * D + dd];
        const float o2 = part_o[(row * P_stride + p + 2) * D + dd], o3 = part_o[(row * P_stride + p + 3) * D + dd];
        acc += s_w[p] * o0;
        acc += s_w[p + 1] * o1;
        acc += s_w[p + 2] * o2;
        acc += s_w[p + 3] * o3;
    }
    for (; p < P; ++p) acc += s_w[p] * part_o[(row * P_stride + p) * D + dd];
    Elem<T>::store(O, row * D + dd, acc / l);
    if (lse != nullptr && dd == 0) lse[row] = m + logf(l);
}

// Chunks per workgroup of attn_decode_mfma_kernel (128 keys each): enough
// for one workgroup per resident slot (two per CU) over the largest key count
// a query may have, so each workgroup streams for long and its set-up and
// merge are spread over many chunks.  (Measured on 32 decode queries with
// 1,000-2,048 memory rows and 2,048 local keys: 105 us at two workgroups per
// CU, 113 us at four, 124 us at eight.)
constexpr int kDecodeWgsPerCu = 2;

struct DecodePlan {
    int nc, P;
};

DecodePlan decode_plan(int64_t B, int Tq, int Hkv, int64_t max_rows, int L, int num_cus) {
    const int64_t chunks = ceil_div(max_rows + L, int64_t(kDecodeChunk));
    const int64_t total = B * Tq * Hkv * chunks;
    int64_t nc = ceil_div(total, int64_t(num_cus) * kDecodeWgsPerCu);
    nc = nc < 1 ? 1 : (nc > chunks ? chunks : nc);
    return DecodePlan{int(nc), int(ceil_div(chunks, nc))};
}

bool decode_applicable(msa_dtype dt, int D, int Hq, int Hkv, int64_t max_rows, int L) {
    const int G = Hq / Hkv;
    return dt == MSA_BF16 && D == 128 && (G == 1 || G == 2 || G == 4 || G == 8) &&
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
                       part_o, part_ml, P, static_cast<T*>(a.O), a.lse, CombineTrim{});
    return hipGetLastError();
}

hipError_t launch_decode(const AttnArgs& a, float* part_o, float2* part_ml, DecodePlan pl, hipStream_t st) {
    hipError_t err = launch_decode_mfma(a, part_o, part_ml, pl.P, pl.nc, st);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((attn_combine_kernel<bf16_t, 128>), dim3(unsigned(a.B * a.Tq * a.Hq)), dim3(128), 0, st,
                       part_o, part_ml, pl.P, static_cast<bf16_t*>(a.O), a.lse, CombineTrim{});
    return hipGetLastError();
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

// ---------------------------------------------------------------- gather + attention
//
// Decode rows on the matrix-core path: the device gather's copy and the
// attention over the local keys run in one launch (the local keys need none
// of the gathered rows), then the attention over the gathered memory rows,
// then one combine over both sets of partials.  Other shapes run the gather
// and then the attention, one after the other.

namespace {

struct GatherAttnPlan {
    bool fused, one;
    int attn_rows;           // > 0: the one-query copy forms the memory rows' partials, this many rows each
    int n_copy;              // copy workgroups
    DecodePlan loc, mem;     // mem.P == 0: no launch over the memory rows
    int P_total;
};

GatherAttnPlan gather_attn_plan(const AttnArgs& a, int64_t cap_rows) {
    GatherAttnPlan g{false, false, 0, kCopyWgs, {0, 0}, {0, 0}, 0};
    if (!decode_applicable(a.dt, a.D, a.Hq, a.Hkv, a.max_rows, a.L) || attn_mfma_applicable(a)) return g;
    g.loc = decode_plan(a.B, a.Tq, a.Hkv, 0, a.L, a.num_cus);
    g.one = a.B == 1 && cap_rows <= kOneMaxRows;
    if (g.one) {
        // a one-token query with at most 8 KV heads (a row of at most 256
        // 16-byte units): the copy workgroups attend over their own rows, 4
        // each while their partials fit the combine, else 8
        int64_t n = ceil_div(cap_rows, int64_t(kOneRows));
        if (a.Tq == 1 && a.Hkv <= 8 && a.max_rows > 0) {
            for (const int R : {kOneAttnRowsFew, kOneAttnRowsMany}) {
                const int64_t w = ceil_div(cap_rows, int64_t(R));
                if (g.loc.P + (w > 0 ? w : 1) <= kMaxParts) {
                    g.attn_rows = R;
                    n = w;
                    break;
                }
            }
        }
        g.n_copy = int(n > 0 ? n : 1);
    }
    if (g.attn_rows > 0) {
        g.P_total = g.loc.P + g.n_copy;
    } else {
        if (a.max_rows > 0) g.mem = decode_plan(a.B, a.Tq, a.Hkv, a.max_rows, 0, a.num_cus);
        g.P_total = g.loc.P + g.mem.P;
    }
    if (g.P_total > kMaxParts) return g;                     // the combine's bound
    g.fused = true;
    return g;
}

size_t partial_bytes(int64_t rows, int D) {
    return align256(size_t(rows) * D * sizeof(float)) + align256(size_t(rows) * sizeof(float2));
}

}  // namespace

size_t gather_attn_workspace(const AttnArgs& a, int64_t cap_rows) {
    const size_t gws = align256(gather_device_workspace(a.B, cap_rows));
    const GatherAttnPlan g = gather_attn_plan(a, cap_rows);
    if (g.fused) return gws + partial_bytes(a.B * a.Tq * a.Hq * g.P_total, a.D);
    return gws + attn_workspace(a.dt, a.B, a.Tq, a.Hq, a.Hkv, a.D, a.max_rows, a.L, a.num_cus);
}

hipError_t launch_gather_attn(const GatherAttnArgs& ga, hipStream_t st) {
    const AttnArgs& a0 = ga.a;
    if (a0.B == 0) return hipSuccess;
    const size_t gws = align256(gather_device_workspace(a0.B, ga.cap_rows));
    AttnArgs a = a0;
    a.ws = static_cast<char*>(a0.ws) + gws;
    a.ws_bytes = a0.ws_bytes - gws;
    const GatherAttnPlan g = gather_attn_plan(a, ga.cap_rows);
    hipError_t err;
    if (!g.fused) {
        err = launch_gather_device(ga.host, ga.row_bytes, ga.n_rows_host, ga.off, ga.n_docs, ga.ids, a.B, ga.K, ga.dst,
                                   ga.cap_rows, ga.mem_off, a0.ws, st);
        if (err != hipSuccess) return err;
        return launch_attn(a, st);
    }
    GatherCopyArgs gc{static_cast<const u32x4*>(ga.host), int64_t(ga.row_bytes / 16), nullptr, int(a.B), ga.ids, ga.K,
                      ga.off, ga.n_docs, ga.n_rows_host, ga.cap_rows, ga.mem_off, static_cast<u32x4*>(ga.dst)};
    if (!g.one) {
        int64_t* src_of_row = nullptr;
        err = launch_gather_plan(ga.ids, a.B, ga.K, ga.off, ga.n_docs, ga.n_rows_host, ga.cap_rows, ga.mem_off, a0.ws,
                                 &src_of_row, st);
        if (err != hipSuccess) return err;
        gc.src_of_row = src_of_row;
    }
    const size_t rows = size_t(a.B) * a.Tq * a.Hq * g.P_total;
    float* part_o = static_cast<float*>(a.ws);
    float2* part_ml = reinterpret_cast<float2*>(static_cast<char*>(a.ws) + align256(rows * a.D * sizeof(float)));
    err = launch_gather_local_attn(gc, g.one, g.attn_rows, g.n_copy, a, part_o, part_ml, g.loc.P, g.loc.nc,
                                   g.P_total, st);
    if (err != hipSuccess) return err;
    if (g.mem.P > 0) {
        err = launch_decode_mfma_mem(a, part_o, part_ml, g.mem.P, g.mem.nc, g.loc.P, g.P_total, st);
        if (err != hipSuccess) return err;
    }
    const CombineTrim tr = g.attn_rows > 0 ? CombineTrim{1, ga.mem_off, g.loc.P, g.attn_rows}
                                           : CombineTrim{0, nullptr, 0, 1};
    hipLaunchKernelGGL((attn_combine_kernel<bf16_t, 128>), dim3(unsigned(a.B * a.Tq * a.Hq)), dim3(128), 0, st,
                       part_o, part_ml, g.P_total, static_cast<bf16_t*>(a.O), a.lse, tr);
    return hipGetLastError();
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
