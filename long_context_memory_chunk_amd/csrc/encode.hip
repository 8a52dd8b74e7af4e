// Stage 1 (offline): document-wise RoPE + chunk mean pooling.
//
// Source: news.neo-ai.one MSA article, 全体設計 › アーキテクチャ (Fig. 2):
// document latent states (K, V, Kr) are compressed by chunk-wise mean
// pooling, and positions restart at 0 in every document; 推論パイプライン
// (Fig. 3), first stage: the pooled (K̄, V̄, K̄r) are cached.
// ruixiangma.github.io blog, 方法 › 稀疏注意力机制 and 文档级RoPE.
//
// Mapping (HBM-bound: every input byte is read once, 3/c of it written):
//   one workgroup per document, 4 waves; wave w pools chunks w, w+4, ...;
//   a lane owns a 16-byte slot of the first half of a head and the matching
//   slot of the second half (the RoPE pair i, i + d/2) of K, V and Kr, and
//   accumulates the chunk's rows in fp32 registers.  Row loads of one wave
//   cover whole 128-byte segments.  cos/sin come from the context's table
//   (float64 angles rounded to float32).
#include "common.hpp"
#include "launch.hpp"

namespace msa {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(256) void encode_pool_kernel(
    const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ Kr,
    const int64_t* __restrict__ tok_off, const int64_t* __restrict__ chunk_off,
    int64_t T_rows, int64_t N, int hkv, int chunk_len,
    const float2* __restrict__ rope_cs, int max_pos,
    T* __restrict__ KVbar, T* __restrict__ Krbar) {
    constexpr int VEC = Vec16<T>::kN;           // elements per 16-byte slot
    constexpr int HALF = D / 2;
    constexpr int SLOTS_PER_HEAD = HALF / VEC;
    const int64_t doc = blockIdx.x;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;

    int64_t s = tok_off[doc], e = tok_off[doc + 1];
    s = s < 0 ? 0 : (s > T_rows ? T_rows : s);
    e = e < s ? s : (e > T_rows ? T_rows : e);
    int64_t c0 = chunk_off[doc], c1 = chunk_off[doc + 1];
    c0 = c0 < 0 ? 0 : (c0 > N ? N : c0);
    c1 = c1 < c0 ? c0 : (c1 > N ? N : c1);
    const int64_t n_chunks_len = (e - s + chunk_len - 1) / chunk_len;
    const int64_t n_chunks = (c1 - c0) < n_chunks_len ? (c1 - c0) : n_chunks_len;

    const int slots = hkv * SLOTS_PER_HEAD;
    const int64_t row_elems = int64_t(hkv) * D;

    for (int64_t j = wave; j < n_chunks; j += 4) {
        const int64_t r0 = s + j * chunk_len;
        const int64_t r1 = (r0 + chunk_len < e) ? r0 + chunk_len : e;
        const float cnt = float(r1 - r0);
        const int64_t n = c0 + j;
        for (int slot = lane; slot < slots; slot += kWave) {
            const int h = slot / SLOTS_PER_HEAD;
            const int i0 = (slot % SLOTS_PER_HEAD) * VEC;
            float k1[VEC], k2[VEC], v1[VEC], v2[VEC], r1_[VEC], r2_[VEC];
#pragma unroll
            for (int u = 0; u < VEC; ++u) { k1[u] = k2[u] = v1[u] = v2[u] = r1_[u] = r2_[u] = 0.f; }
            for (int64_t r = r0; r < r1; ++r) {
                int pos = int(r - s);
                pos = pos < max_pos ? pos : max_pos - 1;
                const int64_t base = r * row_elems + int64_t(h) * D + i0;
                float a[VEC], b[VEC], x[VEC];
                Vec16<T>::load(K + base, a);
                Vec16<T>::load(K + base + HALF, b);
                const float2* cs = rope_cs + int64_t(pos) * HALF + i0;
#pragma unroll
                for (int u = 0; u < VEC; ++u) {
                    const float2 t = cs[u];
                    k1[u] += a[u] * t.x - b[u] * t.y;
                    k2[u] += b[u] * t.x + a[u] * t.y;
                }
                Vec16<T>::load(V + base, x);
#pragma unroll
                for (int u = 0; u < VEC; ++u) v1[u] += x[u];
                Vec16<T>::load(V + base + HALF, x);
#pragma unroll
                for (int u = 0; u < VEC; ++u) v2[u] += x[u];
                Vec16<T>::load(Kr + base, x);
#pragma unroll
                for (int u = 0; u < VEC; ++u) r1_[u] += x[u];
                Vec16<T>::load(Kr + base + HALF, x);
#pragma unroll
                for (int u = 0; u < VEC; ++u) r2_[u] += x[u];
            }
#pragma unroll
            for (int u = 0; u < VEC; ++u) {
                k1[u] /= cnt; k2[u] /= cnt;
                v1[u] /= cnt; v2[u] /= cnt;
                r1_[u] /= cnt; r2_[u] /= cnt;
            }
            T* kv = KVbar + n * 2 * row_elems + int64_t(h) * D + i0;
            Vec16<T>::store(kv, k1);
            Vec16<T>::store(kv + HALF, k2);
            Vec16<T>::store(kv + row_elems, v1);
            Vec16<T>::store(kv + row_elems + HALF, v2);
            T* kr = Krbar + n * row_elems + int64_t(h) * D + i0;
            Vec16<T>::store(kr, r1_);
            Vec16<T>::store(kr + HALF, r2_);
        }
    }
}

template <typename T, int D>
hipError_t launch_typed(const msa_ctx* ctx, const void* K, const void* V, const void* Kr,
                        const int64_t* tok_off, const int64_t* chunk_off, int64_t n_docs,
                        int64_t T_rows, int64_t N, int hkv, int chunk_len, void* KVbar,
                        void* Krbar, hipStream_t st) {
    hipLaunchKernelGGL((encode_pool_kernel<T, D>), dim3(unsigned(n_docs)), dim3(256), 0, st,
                       static_cast<const T*>(K), static_cast<const T*>(V),
                       static_cast<const T*>(Kr), tok_off, chunk_off, T_rows, N, hkv,
                       chunk_len, ctx->rope_cs, ctx->max_pos, static_cast<T*>(KVbar),
                       static_cast<T*>(Krbar));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_encode(const msa_ctx* ctx, msa_dtype dt, const void* K, const void* V,
                         const void* Kr, const int64_t* tok_off, const int64_t* chunk_off,
                         int64_t n_docs, int64_t T_rows, int64_t N, int hkv, int chunk_len,
                         void* KVbar, void* Krbar, hipStream_t st) {
    if (n_docs == 0) return hipSuccess;
    if (dt == MSA_BF16) {
        if (ctx->head_dim == 128)
            return launch_typed<bf16_t, 128>(ctx, K, V, Kr, tok_off, chunk_off, n_docs, T_rows, N,
                                             hkv, chunk_len, KVbar, Krbar, st);
        return launch_typed<bf16_t, 64>(ctx, K, V, Kr, tok_off, chunk_off, n_docs, T_rows, N, hkv,
                                        chunk_len, KVbar, Krbar, st);
    }
    if (ctx->head_dim == 128)
        return launch_typed<float, 128>(ctx, K, V, Kr, tok_off, chunk_off, n_docs, T_rows, N, hkv,
                                        chunk_len, KVbar, Krbar, st);
    return launch_typed<float, 64>(ctx, K, V, Kr, tok_off, chunk_off, n_docs, T_rows, N, hkv,
                                   chunk_len, KVbar, Krbar, st);
}

}  // namespace msa
