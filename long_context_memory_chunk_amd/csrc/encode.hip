// Stage 1 (offline): document-wise RoPE + chunk mean pooling.
//
// Source: news.neo-ai.one MSA article, 全体設計 › アーキテクチャ (Fig. 2):
// document latent states (K, V, Kr) are compressed by chunk-wise mean
// pooling, and positions restart at 0 in every document; 推論パイプライン
// (Fig. 3), first stage: the pooled (K̄, V̄, K̄r) are cached.
// ruixiangma.github.io blog, 方法 › 稀疏注意力机制 and 文档级RoPE.
//
// Mapping (HBM-bound: every input byte is read once, 3/c of it written):
//   one wave per pooled chunk over the whole bank (grid-stride), so a long
//   document costs no more per wave than a short one; the wave finds its
//   document by binary search in doc_chunk_off.  A lane owns a 16-byte slot
//   of the first half of a head and the matching slot of the second half (the
//   RoPE pair i, i + d/2) of K, V and Kr, and accumulates the chunk's rows in
//   fp32 registers, in row order.  Rows are taken UNROLL at a time with all of
//   their loads issued first (nontemporal: the raw tensors are streamed once),
//   which keeps enough bytes in flight per wave to cover HBM latency.  Row
//   loads of one wave cover whole 128-byte segments.  cos/sin come from the
//   context's table (float64 angles rounded to float32).  The host has
//   checked that the longest document (max_doc_len) fits the table; a
//   document the device offsets make longer than that gets NaN rows instead
//   of clamped positions, so a wrong length is visible and never read past
//   the table.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace msa {
namespace {

constexpr int kEncodeUnroll = 1;   // deeper unrolling measured no faster (bytes in flight per CU stay ~90 KB)

template <typename T> struct Raw16;
template <> struct Raw16<float> {
    __device__ __forceinline__ static void unpack(const u32x4& v, float* out) {
        out[0] = __uint_as_float(v[0]); out[1] = __uint_as_float(v[1]);
        out[2] = __uint_as_float(v[2]); out[3] = __uint_as_float(v[3]);
    }
};
template <> struct Raw16<bf16_t> {
    __device__ __forceinline__ static void unpack(const u32x4& v, float* out) {
        out[0] = bf16_lo(v[0]); out[1] = bf16_hi(v[0]);
        out[2] = bf16_lo(v[1]); out[3] = bf16_hi(v[1]);
        out[4] = bf16_lo(v[2]); out[5] = bf16_hi(v[2]);
        out[6] = bf16_lo(v[3]); out[7] = bf16_hi(v[3]);
    }
};

__device__ __forceinline__ u32x4 ld_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Largest d in [0, n_docs) with off[d] <= n (off non-decreasing, off[0] = 0).
__device__ __forceinline__ int64_t doc_of_chunk(const int64_t* __restrict__ off, int64_t n_docs,
                                                int64_t n) {
    int64_t lo = 0, hi = n_docs - 1;
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if (off[mid] <= n) lo = mid; else hi = mid - 1;
    }
    return lo;
}

template <typename T, int D, int UNROLL>
__global__ __launch_bounds__(256) void encode_pool_kernel(
    const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ Kr,
    const int64_t* __restrict__ tok_off, const int64_t* __restrict__ chunk_off, int64_t n_docs,
    int64_t T_rows, int64_t N, int hkv, int chunk_len,
    const float2* __restrict__ rope_cs, int64_t max_doc_len,
    T* __restrict__ KVbar, T* __restrict__ Krbar) {
    constexpr int VEC = Vec16<T>::kN;           // elements per 16-byte slot
    constexpr int HALF = D / 2;
    constexpr int SLOTS_PER_HEAD = HALF / VEC;
    const int lane = threadIdx.x % kWave;
    const int slots = hkv * SLOTS_PER_HEAD;
    const int64_t row_elems = int64_t(hkv) * D;
    const int64_t n_waves = int64_t(gridDim.x) * (blockDim.x / kWave);

    for (int64_t n = int64_t(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave; n < N;
         n += n_waves) {
        const int64_t doc = doc_of_chunk(chunk_off, n_docs, n);
        int64_t s = tok_off[doc], e = tok_off[doc + 1];
        s = s < 0 ? 0 : (s > T_rows ? T_rows : s);
        e = e < s ? s : (e > T_rows ? T_rows : e);
        const int64_t j = n - chunk_off[doc];
        const int64_t r0 = s + j * chunk_len;
        if (j < 0 || r0 >= e) continue;         // inconsistent offsets: row n is left unwritten
        const int64_t r1 = (r0 + chunk_len < e) ? r0 + chunk_len : e;
        const float cnt = float(r1 - r0);
        if (e - s > max_doc_len) {              // longer than the host was told: NaN, not clamped positions
            float nan[VEC];
#pragma unroll
            for (int u = 0; u < VEC; ++u) nan[u] = __builtin_nanf("");
            for (int slot = lane; slot < 2 * slots; slot += kWave) {
                const int64_t o = int64_t(slot) * VEC;
                Vec16<T>::store(KVbar + n * 2 * row_elems + o, nan);
                Vec16<T>::store(KVbar + n * 2 * row_elems + row_elems + o, nan);
            }
            for (int slot = lane; slot < 2 * slots; slot += kWave)
                Vec16<T>::store(Krbar + n * row_elems + int64_t(slot) * VEC, nan);
            continue;
        }

        for (int slot = lane; slot < slots; slot += kWave) {
            const int h = slot / SLOTS_PER_HEAD;
            const int i0 = (slot % SLOTS_PER_HEAD) * VEC;
            float k1[VEC], k2[VEC], v1[VEC], v2[VEC], q1[VEC], q2[VEC];
#pragma unroll
            for (int u = 0; u < VEC; ++u) { k1[u] = k2[u] = v1[u] = v2[u] = q1[u] = q2[u] = 0.f; }
            const T* kp = K + r0 * row_elems + int64_t(h) * D + i0;
            const T* vp = V + r0 * row_elems + int64_t(h) * D + i0;
            const T* qp = Kr + r0 * row_elems + int64_t(h) * D + i0;
            int64_t r = r0;
            auto rows = [&](auto n_rows_c) {
                constexpr int R = decltype(n_rows_c)::value;
                u32x4 ka[R], kb[R], va[R], vb[R], qa[R], qb[R];
#pragma unroll
                for (int u = 0; u < R; ++u) {
                    const int64_t o = int64_t(u) * row_elems;
                    ka[u] = ld_stream(kp + o); kb[u] = ld_stream(kp + o + HALF);
                    va[u] = ld_stream(vp + o); vb[u] = ld_stream(vp + o + HALF);
                    qa[u] = ld_stream(qp + o); qb[u] = ld_stream(qp + o + HALF);
                }
#pragma unroll
                for (int u = 0; u < R; ++u) {
                    const int64_t pos = r + u - s;    // < e - s <= max_doc_len <= max_pos
                    const float2* cs = rope_cs + pos * HALF + i0;
                    float a[VEC], b[VEC];
                    Raw16<T>::unpack(ka[u], a);
                    Raw16<T>::unpack(kb[u], b);
#pragma unroll
                    for (int w = 0; w < VEC; ++w) {
                        const float2 t = cs[w];
                        k1[w] += a[w] * t.x - b[w] * t.y;
                        k2[w] += b[w] * t.x + a[w] * t.y;
                    }
                    Raw16<T>::unpack(va[u], a);
                    Raw16<T>::unpack(vb[u], b);
#pragma unroll
                    for (int w = 0; w < VEC; ++w) { v1[w] += a[w]; v2[w] += b[w]; }
                    Raw16<T>::unpack(qa[u], a);
                    Raw16<T>::unpack(qb[u], b);
#pragma unroll
                    for (int w = 0; w < VEC; ++w) { q1[w] += a[w]; q2[w] += b[w]; }
                }
                kp += R * row_elems; vp += R * row_elems; qp += R * row_elems;
                r += R;
            };
            while (r + UNROLL <= r1) rows(std::integral_constant<int, UNROLL>{});
            while (r < r1) rows(std::integral_constant<int, 1>{});
#pragma unroll
            for (int u = 0; u < VEC; ++u) {
                k1[u] /= cnt; k2[u] /= cnt;
                v1[u] /= cnt; v2[u] /= cnt;
                q1[u] /= cnt; q2[u] /= cnt;
            }
            T* kv = KVbar + n * 2 * row_elems + int64_t(h) * D + i0;
            Vec16<T>::store(kv, k1);
            Vec16<T>::store(kv + HALF, k2);
            Vec16<T>::store(kv + row_elems, v1);
            Vec16<T>::store(kv + row_elems + HALF, v2);
            T* kr = Krbar + n * row_elems + int64_t(h) * D + i0;
            Vec16<T>::store(kr, q1);
            Vec16<T>::store(kr + HALF, q2);
        }
    }
}

// 16-byte streaming store of VEC floats converted to T (the token-row
// gradients are written once and not read again here).
template <typename T> struct St16;
template <> struct St16<float> {
    __device__ __forceinline__ static void put(float* p, const float* in) {
        const u32x4 v = {__float_as_uint(in[0]), __float_as_uint(in[1]), __float_as_uint(in[2]),
                         __float_as_uint(in[3])};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
    }
};
template <> struct St16<bf16_t> {
    __device__ __forceinline__ static void put(bf16_t* p, const float* in) {
        const u32x4 v = {pack_bf16x2(in[0], in[1]), pack_bf16x2(in[2], in[3]), pack_bf16x2(in[4], in[5]),
                         pack_bf16x2(in[6], in[7])};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
    }
};

// Backward of the pooling: every token row of a chunk gets 1/count of the
// chunk's gradient, the key part turned back by the row's document-local
// angle.  Same mapping as the forward (one wave per chunk, a lane owning a
// 16-byte slot of each RoPE half): the pooled gradient row is read once and
// the chunk's token rows are written.
template <typename T, int D>
__global__ __launch_bounds__(256) void encode_bwd_kernel(
    const T* __restrict__ dKVbar, const T* __restrict__ dKrbar, const int64_t* __restrict__ tok_off,
    const int64_t* __restrict__ chunk_off, int64_t n_docs, int64_t T_rows, int64_t N, int hkv, int chunk_len,
    const float2* __restrict__ rope_cs, int64_t max_doc_len, T* __restrict__ dK, T* __restrict__ dV,
    T* __restrict__ dKr) {
    constexpr int VEC = Vec16<T>::kN;
    constexpr int HALF = D / 2;
    constexpr int SLOTS_PER_HEAD = HALF / VEC;
    const int lane = threadIdx.x % kWave;
    const int slots = hkv * SLOTS_PER_HEAD;
    const int64_t row_elems = int64_t(hkv) * D;
    const int64_t n_waves = int64_t(gridDim.x) * (blockDim.x / kWave);

    for (int64_t n = int64_t(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave; n < N;
         n += n_waves) {
        const int64_t doc = doc_of_chunk(chunk_off, n_docs, n);
        int64_t s = tok_off[doc], e = tok_off[doc + 1];
        s = s < 0 ? 0 : (s > T_rows ? T_rows : s);
        e = e < s ? s : (e > T_rows ? T_rows : e);
        const int64_t j = n - chunk_off[doc];
        const int64_t r0 = s + j * chunk_len;
        if (j < 0 || r0 >= e) continue;         // inconsistent offsets: nothing is written
        const int64_t r1 = (r0 + chunk_len < e) ? r0 + chunk_len : e;
        const float inv = 1.f / float(r1 - r0);
        const bool too_long = e - s > max_doc_len;   // NaN gradients, not clamped positions

        for (int slot = lane; slot < slots; slot += kWave) {
            const int h = slot / SLOTS_PER_HEAD;
            const int i0 = (slot % SLOTS_PER_HEAD) * VEC;
            float k1[VEC], k2[VEC], v1[VEC], v2[VEC], q1[VEC], q2[VEC];
            const T* kv = dKVbar + n * 2 * row_elems + int64_t(h) * D + i0;
            const T* kr = dKrbar + n * row_elems + int64_t(h) * D + i0;
            Vec16<T>::load(kv, k1);
            Vec16<T>::load(kv + HALF, k2);
            Vec16<T>::load(kv + row_elems, v1);
            Vec16<T>::load(kv + row_elems + HALF, v2);
            Vec16<T>::load(kr, q1);
            Vec16<T>::load(kr + HALF, q2);
#pragma unroll
            for (int u = 0; u < VEC; ++u) {
                k1[u] *= inv; k2[u] *= inv;
                v1[u] *= inv; v2[u] *= inv;
                q1[u] *= inv; q2[u] *= inv;
            }
            if (too_long) {
#pragma unroll
                for (int u = 0; u < VEC; ++u) k1[u] = k2[u] = v1[u] = v2[u] = q1[u] = q2[u] = __builtin_nanf("");
            }
            for (int64_t r = r0; r < r1; ++r) {
                float a[VEC], bb[VEC];
                if (too_long) {
#pragma unroll
                    for (int w = 0; w < VEC; ++w) a[w] = bb[w] = k1[w];
                } else {
                    const int64_t pos = r - s;          // < e - s <= max_doc_len <= max_pos
                    const float2* cs = rope_cs + pos * HALF + i0;
#pragma unroll
                    for (int w = 0; w < VEC; ++w) {
                        const float2 t = cs[w];
                        a[w] = k1[w] * t.x + k2[w] * t.y;     // the transpose of the rotation
                        bb[w] = k2[w] * t.x - k1[w] * t.y;
                    }
                }
                const int64_t o = r * row_elems + int64_t(h) * D + i0;
                St16<T>::put(dK + o, a);
                St16<T>::put(dK + o + HALF, bb);
                St16<T>::put(dV + o, v1);
                St16<T>::put(dV + o + HALF, v2);
                St16<T>::put(dKr + o, q1);
                St16<T>::put(dKr + o + HALF, q2);
            }
        }
    }
}

template <typename T, int D>
hipError_t launch_bwd_typed(const msa_ctx* ctx, const void* dKVbar, const void* dKrbar, const int64_t* tok_off,
                            const int64_t* chunk_off, int64_t n_docs, int64_t T_rows, int64_t N, int hkv,
                            int chunk_len, int64_t max_doc_len, void* dK, void* dV, void* dKr, hipStream_t st) {
    const int64_t blocks = ceil_div(N, int64_t(4));
    const unsigned grid = unsigned(blocks < (int64_t(1) << 30) ? blocks : (int64_t(1) << 30));
    hipLaunchKernelGGL((encode_bwd_kernel<T, D>), dim3(grid), dim3(256), 0, st, static_cast<const T*>(dKVbar),
                       static_cast<const T*>(dKrbar), tok_off, chunk_off, n_docs, T_rows, N, hkv, chunk_len,
                       ctx->rope_cs, max_doc_len, static_cast<T*>(dK), static_cast<T*>(dV), static_cast<T*>(dKr));
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_typed(const msa_ctx* ctx, const void* K, const void* V, const void* Kr,
                        const int64_t* tok_off, const int64_t* chunk_off, int64_t n_docs,
                        int64_t T_rows, int64_t N, int hkv, int chunk_len, int64_t max_doc_len,
                        void* KVbar, void* Krbar, hipStream_t st) {
    const int64_t blocks = ceil_div(N, int64_t(4));
    const unsigned grid = unsigned(blocks < (int64_t(1) << 30) ? blocks : (int64_t(1) << 30));
    hipLaunchKernelGGL((encode_pool_kernel<T, D, kEncodeUnroll>), dim3(grid), dim3(256), 0, st,
                       static_cast<const T*>(K), static_cast<const T*>(V),
                       static_cast<const T*>(Kr), tok_off, chunk_off, n_docs, T_rows, N, hkv,
                       chunk_len, ctx->rope_cs, max_doc_len, static_cast<T*>(KVbar),
                       static_cast<T*>(Krbar));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_encode(const msa_ctx* ctx, msa_dtype dt, const void* K, const void* V,
                         const void* Kr, const int64_t* tok_off, const int64_t* chunk_off,
                         int64_t n_docs, int64_t T_rows, int64_t N, int hkv, int chunk_len,
                         int64_t max_doc_len, void* KVbar, void* Krbar, hipStream_t st) {
    if (n_docs == 0 || N == 0) return hipSuccess;
    if (dt == MSA_BF16) {
        if (ctx->head_dim == 128)
            return launch_typed<bf16_t, 128>(ctx, K, V, Kr, tok_off, chunk_off, n_docs, T_rows, N,
                                             hkv, chunk_len, max_doc_len, KVbar, Krbar, st);
        return launch_typed<bf16_t, 64>(ctx, K, V, Kr, tok_off, chunk_off, n_docs, T_rows, N, hkv,
                                        chunk_len, max_doc_len, KVbar, Krbar, st);
    }
    if (ctx->head_dim == 128)
        return launch_typed<float, 128>(ctx, K, V, Kr, tok_off, chunk_off, n_docs, T_rows, N, hkv,
                                        chunk_len, max_doc_len, KVbar, Krbar, st);
    return launch_typed<float, 64>(ctx, K, V, Kr, tok_off, chunk_off, n_docs, T_rows, N, hkv,
                                   chunk_len, max_doc_len, KVbar, Krbar, st);
}

}  // namespace msa

namespace msa {

hipError_t launch_encode_bwd(const msa_ctx* ctx, msa_dtype dt, const void* dKVbar, const void* dKrbar,
                             const int64_t* tok_off, const int64_t* chunk_off, int64_t n_docs, int64_t T_rows,
                             int64_t N, int hkv, int chunk_len, int64_t max_doc_len, void* dK, void* dV,
                             void* dKr, hipStream_t st) {
    if (n_docs == 0 || N == 0) return hipSuccess;
    if (dt == MSA_BF16)
        return ctx->head_dim == 128
                   ? launch_bwd_typed<bf16_t, 128>(ctx, dKVbar, dKrbar, tok_off, chunk_off, n_docs, T_rows, N, hkv,
                                                   chunk_len, max_doc_len, dK, dV, dKr, st)
                   : launch_bwd_typed<bf16_t, 64>(ctx, dKVbar, dKrbar, tok_off, chunk_off, n_docs, T_rows, N, hkv,
                                                  chunk_len, max_doc_len, dK, dV, dKr, st);
    return ctx->head_dim == 128
               ? launch_bwd_typed<float, 128>(ctx, dKVbar, dKrbar, tok_off, chunk_off, n_docs, T_rows, N, hkv,
                                              chunk_len, max_doc_len, dK, dV, dKr, st)
               : launch_bwd_typed<float, 64>(ctx, dKVbar, dKrbar, tok_off, chunk_off, n_docs, T_rows, N, hkv,
                                             chunk_len, max_doc_len, dK, dV, dKr, st);
}

}  // namespace msa
