// Backward of the stage 2a document score: gradients of the routing query Qr
// and the pooled routing keys K̄r from a gradient of the loss with respect to
// the document scores.
//
// Sources: ruixiangma.github.io blog, 训练策略 (continued pre-training adds an
// auxiliary routing loss, a supervised contrastive loss that separates relevant
// from irrelevant document blocks, to the generation loss; it trains the
// router through the document scores); the score differentiated is that of
// news.neo-ai.one MSA article, 全体設計 › アーキテクチャ (Fig. 2): cosine of Qr
// and K̄r averaged over heads, max over query tokens and the document's chunks.
//
// score[b, doc] = max over chunks n of doc and tokens t of
//                 (1/Hq) sum_h cos(Qr[b,t,h], K̄r[n, h/G]),
// cos(q, k) = q.k / (max(|q|, eps) max(|k|, eps)).  The max passes its
// gradient to its arg max (n*, t*) only (ties: lowest chunk, then lowest token);
// with w = dscore[b, doc] / Hq and c_h the cosine of head h there,
//   dQr[b,t*,h] += w (k^ - c_h q^_h) / |q_h|      (w k^ / eps if |q_h| <= eps)
//   dK̄r[n*,g]   += w sum_{h in g} (q^_h - c_h k^) / |k|   (w sum q^_h / eps if |k| <= eps)
// where ^ divides by the clamped norm.
//
// Kernels:
//   route_prep (route_scan.hip)  U[b,t,g] = sum_{h in g} q^_h, fp32.
//   rbwd_knorm     |K̄r[n, g]| for every chunk row and KV head.
//   rbwd_chunkmax  every (token, chunk) score (the group fold of the forward,
//                  U . k^ / Hq, in fp32 on the vector units) and, per chunk,
//                  the best token as one 64-bit key (score, then lowest token).
//   rbwd_docmax    per (b, doc) with a non-zero gradient: the best chunk key
//                  (lowest chunk among equal scores), then the per-head
//                  cosines at the arg max.
//   rbwd_dq        one workgroup per (b, t): the documents whose arg max token
//                  is t, in document order, summed into dQr[b, t].
//   rbwd_dk        one workgroup per document: for each of its chunks, the
//                  queries whose arg max chunk it is, in query order, summed
//                  into dK̄r[n] (zero rows for chunks that got nothing).
// Every sum runs in a fixed order (no atomics): the result does not depend on
// scheduling.
#include "launch.hpp"
#include "route_scan.hpp"

namespace msa {
namespace {

constexpr float kEps = 1e-8f;

// Monotone map of a float to an unsigned integer (finite inputs).
__device__ __forceinline__ uint32_t order32(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <typename T>
__global__ __launch_bounds__(64) void rbwd_knorm_kernel(const T* __restrict__ Kr, int64_t N, int hkv, int D,
                                                        float* __restrict__ knorm) {
    const int64_t row = blockIdx.x;          // (n, g)
    const int lane = threadIdx.x;
    float s = 0.f;
    for (int c = lane; c < D; c += kWave) {
        const float x = Elem<T>::load(Kr, row * D + c);
        s += x * x;
    }
    s = wave_sum(s);
    if (lane == 0) knorm[row] = sqrtf(s);
}

// Per chunk row n and query b: the best token, as the key
// order32(score) << 32 | (2^32 - 1 - t) (higher score, then lower t, wins).
// A workgroup takes 32 chunk rows and 256 tokens at a time; wave w owns chunk
// rows 8w .. 8w+7 and lane l the tokens l, l+64, l+128, l+192, so each thread
// keeps a 4 x 8 block of scores.  The contraction over the Hkv * D elements
// runs through LDS 32 elements at a time; per 4 elements a thread makes four
// 16-byte token loads (distinct rows, conflict-free) and eight broadcast
// unit-key loads for 128 fp32 multiply-adds.
constexpr int kCB = 32;                       // chunk rows per workgroup (8 per wave)
constexpr int kEB = 32;                       // contraction elements per LDS stage
constexpr int kUS = kEB + 4;                  // padded row of the token stage

template <typename T>
__global__ __launch_bounds__(256) void rbwd_chunkmax_kernel(
    const float* __restrict__ U, int Tq, int Hq, const T* __restrict__ Kr, int64_t N, int hkv, int D,
    const float* __restrict__ knorm, unsigned long long* __restrict__ ckey) {
    __shared__ __attribute__((aligned(16))) float sU[256 * kUS];
    __shared__ __attribute__((aligned(16))) float sK[kCB * kEB];
    const int64_t n0 = int64_t(blockIdx.x) * kCB;
    const int64_t b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int RW = hkv * D;
    const int nb = int(N - n0 < kCB ? N - n0 : kCB);
    const float inv_hq = 1.f / float(Hq);
    unsigned long long best = 0ull;           // lane j < 8: running best of chunk n0 + 8 wave + j
    for (int t0 = 0; t0 < Tq; t0 += 256) {
        float acc[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
        for (int e0 = 0; e0 < RW; e0 += kEB) {
            __syncthreads();                   // every thread done with the previous stage
            for (int i = tid; i < 256 * kEB; i += 256) {
                const int r = i / kEB, c = i % kEB;
                sU[r * kUS + c] = (t0 + r < Tq) ? U[(b * Tq + t0 + r) * int64_t(RW) + e0 + c] : 0.f;
            }
            for (int i = tid; i < kCB * kEB; i += 256) {
                const int j = i / kEB, c = i % kEB;
                float v = 0.f;
                if (j < nb) {
                    const int64_t n = n0 + j;
                    v = Elem<T>::load(Kr, n * RW + e0 + c) / fmaxf(knorm[n * hkv + (e0 + c) / D], kEps);
                }
                sK[i] = v;
            }
            __syncthreads();
#pragma unroll
            for (int c = 0; c < kEB; c += 4) {
                float4 u[4], k[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) u[i] = *reinterpret_cast<const float4*>(sU + (lane + 64 * i) * kUS + c);
#pragma unroll
                for (int j = 0; j < 8; ++j) k[j] = *reinterpret_cast<const float4*>(sK + (8 * wave + j) * kEB + c);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                    {
                        acc[i][j] = fmaf(u[i].x, k[j].x, acc[i][j]);
                        acc[i][j] = fmaf(u[i].y, k[j].y, acc[i][j]);
                        acc[i][j] = fmaf(u[i].z, k[j].z, acc[i][j]);
                        acc[i][j] = fmaf(u[i].w, k[j].w, acc[i][j]);
                    }
            }
        }
        // best token of each of the wave's chunks over this block of tokens
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            unsigned long long key = 0ull;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + lane + 64 * i;
                if (t < Tq) {
                    const unsigned long long kk =
                        (static_cast<unsigned long long>(order32(acc[i][j] * inv_hq)) << 32) | (0xFFFFFFFFu - uint32_t(t));
                    key = kk > key ? kk : key;
                }
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const unsigned long long other = __shfl_xor(key, o);
                key = other > key ? other : key;
            }
            if (lane == j) best = key > best ? key : best;
        }
    }
    const int j = 8 * wave + lane;
    if (lane < 8 && j < nb) ckey[b * N + n0 + j] = best;
}

// Per (b, doc) with a non-zero gradient: the arg max over the document's
// chunks (the first chunk among equal scores) of the per-chunk best keys,
// then the per-head cosines there.
template <typename T>
__global__ __launch_bounds__(64) void rbwd_docmax_kernel(
    const T* __restrict__ Qr, int Tq, int Hq, const T* __restrict__ Kr, int64_t N, int hkv, int D,
    const int64_t* __restrict__ chunk_off, int64_t n_docs, const float* __restrict__ dscore,
    const unsigned long long* __restrict__ ckey, const float* __restrict__ knorm, int2* __restrict__ arg,
    float* __restrict__ cosv) {
    const int64_t doc = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x;
    const int64_t bd = b * n_docs + doc;
    int64_t n_lo = chunk_off[doc], n_hi = chunk_off[doc + 1];
    n_lo = n_lo < 0 ? 0 : (n_lo > N ? N : n_lo);
    n_hi = n_hi < n_lo ? n_lo : (n_hi > N ? N : n_hi);
    if (dscore[bd] == 0.f || n_hi == n_lo) {
        if (lane == 0) arg[bd] = make_int2(-1, -1);
        return;
    }
    // lane-strided scan, then a wave max of (score, -chunk, -token)
    unsigned long long hi = 0ull;             // order32(score) << 32 | ~n_local
    uint32_t tok = 0;
    for (int64_t n = n_lo + lane; n < n_hi; n += kWave) {
        const unsigned long long k = ckey[b * N + n];
        const unsigned long long key = (k & 0xFFFFFFFF00000000ull) | (0xFFFFFFFFu - uint32_t(n - n_lo));
        if (key > hi) {
            hi = key;
            tok = 0xFFFFFFFFu - uint32_t(k & 0xFFFFFFFFull);
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const unsigned long long ok = __shfl_xor(hi, o);
        const uint32_t ot = __shfl_xor(tok, o);
        if (ok > hi) {
            hi = ok;
            tok = ot;
        }
    }
    const int64_t n = n_lo + (0xFFFFFFFFu - uint32_t(hi & 0xFFFFFFFFull));
    const int t = int(tok);
    if (lane == 0) arg[bd] = make_int2(int(n), t);
    const int G = Hq / hkv;
    for (int h = 0; h < Hq; ++h) {
        const int g = h / G;
        float qq = 0.f, qk = 0.f;
        for (int c = lane; c < D; c += kWave) {
            const float q = Elem<T>::load(Qr, ((b * Tq + t) * Hq + h) * int64_t(D) + c);
            const float kv = Elem<T>::load(Kr, (n * hkv + g) * int64_t(D) + c);
            qq += q * q;
            qk += q * kv;
        }
        qq = wave_sum(qq);
        qk = wave_sum(qk);
        if (lane == 0)
            cosv[bd * Hq + h] = qk / (fmaxf(sqrtf(qq), kEps) * fmaxf(knorm[n * hkv + g], kEps));
    }
}

template <typename T>
__global__ __launch_bounds__(256) void rbwd_dq_kernel(
    const T* __restrict__ Qr, int Tq, int Hq, const T* __restrict__ Kr, int hkv, int D, int64_t n_docs,
    const float* __restrict__ dscore, const float* __restrict__ knorm, const int2* __restrict__ arg,
    const float* __restrict__ cosv, float* __restrict__ dQr) {
    extern __shared__ float smem[];
    const int RW = hkv * D;
    float* A = smem;                          // [RW]: sum of w k^ per KV head
    float* C = smem + RW;                     // [Hq]: sum of w c_h
    float* nq = C + Hq;                       // [Hq]: |q_h|
    const int t = blockIdx.x;
    const int64_t b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const float inv_hq = 1.f / float(Hq);
    for (int e = tid; e < RW; e += 256) A[e] = 0.f;
    for (int h = tid; h < Hq; h += 256) C[h] = 0.f;
    const int64_t qbase = (b * Tq + t) * int64_t(Hq) * D;
    for (int h = wave; h < Hq; h += 4) {
        float s = 0.f;
        for (int c = lane; c < D; c += kWave) {
            const float q = Elem<T>::load(Qr, qbase + int64_t(h) * D + c);
            s += q * q;
        }
        s = wave_sum(s);
        if (lane == 0) nq[h] = sqrtf(s);
    }
    // documents whose arg max token is t, 256 at a time, compacted in
    // document order (ballot prefix counts) and then summed in that order
    __shared__ int s_docs[256];
    __shared__ int s_cnt[4];
    for (int64_t d0 = 0; d0 < n_docs; d0 += 256) {
        const int64_t doc = d0 + tid;
        const bool hit = doc < n_docs && arg[b * n_docs + doc].y == t;   // -1: no gradient
        const unsigned long long m = __ballot(hit);
        const int before = __popcll(m & ((1ull << lane) - 1ull));
        __syncthreads();                       // the previous batch's list is consumed
        if (lane == 0) s_cnt[wave] = __popcll(m);
        __syncthreads();
        int off = 0;
        for (int w = 0; w < wave; ++w) off += s_cnt[w];
        if (hit) s_docs[off + before] = int(tid);
        const int total = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
        __syncthreads();
        for (int i = 0; i < total; ++i) {
            const int64_t dd = d0 + s_docs[i];
            const int2 a = arg[b * n_docs + dd];
            const float w = dscore[b * n_docs + dd] * inv_hq;
            for (int e = tid; e < RW; e += 256) {
                const float nk = fmaxf(knorm[int64_t(a.x) * hkv + e / D], kEps);
                A[e] += w * Elem<T>::load(Kr, int64_t(a.x) * RW + e) / nk;
            }
            for (int h = tid; h < Hq; h += 256) C[h] += w * cosv[(b * n_docs + dd) * Hq + h];
        }
    }
    __syncthreads();
    const int G = Hq / hkv;
    for (int e = tid; e < Hq * D; e += 256) {
        const int h = e / D, c = e % D;
        const float n = nq[h];
        const float av = A[(h / G) * D + c];
        float d;
        if (n > kEps) d = (av - C[h] * Elem<T>::load(Qr, qbase + e) / n) / n;
        else d = av / kEps;
        dQr[qbase + e] = d;
    }
}

template <typename T>
__global__ __launch_bounds__(256) void rbwd_dk_kernel(
    const T* __restrict__ Kr, int64_t N, int hkv, int D, int Tq, int Hq, const int64_t* __restrict__ chunk_off,
    int64_t n_docs, int64_t B, const float* __restrict__ dscore, const float* __restrict__ U,
    const float* __restrict__ knorm, const int2* __restrict__ arg, const float* __restrict__ cosv,
    float* __restrict__ dKr) {
    extern __shared__ float smem[];
    const int RW = hkv * D;
    float* A = smem;                          // [RW]: sum of w sum_{h in g} q^_h
    float* C = smem + RW;                     // [hkv]: sum of w sum_{h in g} c_h
    const int64_t doc = blockIdx.x;
    const int tid = threadIdx.x;
    int64_t n_lo = chunk_off[doc], n_hi = chunk_off[doc + 1];
    n_lo = n_lo < 0 ? 0 : (n_lo > N ? N : n_lo);
    n_hi = n_hi < n_lo ? n_lo : (n_hi > N ? N : n_hi);
    const int G = Hq / hkv;
    const float inv_hq = 1.f / float(Hq);
    for (int64_t n = n_lo; n < n_hi; ++n) {
        __syncthreads();
        for (int e = tid; e < RW; e += 256) A[e] = 0.f;
        for (int g = tid; g < hkv; g += 256) C[g] = 0.f;
        __syncthreads();
        for (int64_t b = 0; b < B; ++b) {
            const int2 a = arg[b * n_docs + doc];
            if (a.x != int(n)) continue;
            const float w = dscore[b * n_docs + doc] * inv_hq;
            const float* ur = U + (b * Tq + a.y) * int64_t(RW);
            for (int e = tid; e < RW; e += 256) A[e] += w * ur[e];
            for (int g = tid; g < hkv; g += 256) {
                float cs = 0.f;
                for (int h = g * G; h < (g + 1) * G; ++h) cs += cosv[(b * n_docs + doc) * Hq + h];
                C[g] += w * cs;
            }
        }
        __syncthreads();
        for (int e = tid; e < RW; e += 256) {
            const float nk = knorm[n * hkv + e / D];
            float d;
            if (nk > kEps) d = (A[e] - C[e / D] * Elem<T>::load(Kr, n * RW + e) / nk) / nk;
            else d = A[e] / kEps;
            dKr[n * RW + e] = d;
        }
    }
}

struct RbwdLayout {
    size_t u, kn, arg, cos, ck, total;
};

RbwdLayout rbwd_layout(int64_t B, int Tq, int Hq, int Hkv, int D, int64_t N, int64_t n_docs) {
    RbwdLayout l;
    l.u = align256(size_t(B) * Tq * Hkv * D * sizeof(float));
    l.kn = align256(size_t(N) * Hkv * sizeof(float));
    l.arg = align256(size_t(B) * n_docs * sizeof(int2));
    l.cos = align256(size_t(B) * n_docs * Hq * sizeof(float));
    l.ck = align256(size_t(B) * N * sizeof(unsigned long long));
    l.total = l.u + l.kn + l.arg + l.cos + l.ck;
    return l;
}

template <typename T>
hipError_t launch_rbwd_t(const RouteBwdArgs& a, hipStream_t st) {
    const RouteArgs& r = a.r;
    const RbwdLayout l = rbwd_layout(r.B, r.Tq, r.Hq, r.Hkv, r.D, r.N, r.n_docs);
    char* w = static_cast<char*>(r.ws);
    float* U = reinterpret_cast<float*>(w);
    float* knorm = reinterpret_cast<float*>(w + l.u);
    int2* arg = a.arg_out ? reinterpret_cast<int2*>(a.arg_out) : reinterpret_cast<int2*>(w + l.u + l.kn);
    float* cosv = reinterpret_cast<float*>(w + l.u + l.kn + l.arg);
    unsigned long long* ckey = reinterpret_cast<unsigned long long*>(w + l.u + l.kn + l.arg + l.cos);
    const T* Qr = static_cast<const T*>(r.Qr);
    const T* Kr = static_cast<const T*>(r.Krbar);
    hipError_t err = launch_route_prep(r, U, st);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((rbwd_knorm_kernel<T>), dim3(unsigned(r.N * r.Hkv)), dim3(64), 0, st, Kr, r.N, r.Hkv, r.D,
                       knorm);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((rbwd_chunkmax_kernel<T>), dim3(unsigned(ceil_div(r.N, int64_t(kCB))), unsigned(r.B)),
                       dim3(256), 0, st, U, r.Tq, r.Hq, Kr, r.N, r.Hkv, r.D, knorm, ckey);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((rbwd_docmax_kernel<T>), dim3(unsigned(r.n_docs), unsigned(r.B)), dim3(64), 0, st, Qr, r.Tq,
                       r.Hq, Kr, r.N, r.Hkv, r.D, r.chunk_off, r.n_docs, a.dscore, ckey, knorm, arg, cosv);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const size_t dq_lds = size_t(r.Hkv * r.D + 2 * r.Hq) * sizeof(float);
    hipLaunchKernelGGL((rbwd_dq_kernel<T>), dim3(unsigned(r.Tq), unsigned(r.B)), dim3(256), dq_lds, st, Qr, r.Tq,
                       r.Hq, Kr, r.Hkv, r.D, r.n_docs, a.dscore, knorm, arg, cosv, a.dQr);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const size_t dk_lds = size_t(r.Hkv * r.D + r.Hkv) * sizeof(float);
    hipLaunchKernelGGL((rbwd_dk_kernel<T>), dim3(unsigned(r.n_docs)), dim3(256), dk_lds, st, Kr, r.N, r.Hkv, r.D,
                       r.Tq, r.Hq, r.chunk_off, r.n_docs, r.B, a.dscore, U, knorm, arg, cosv, a.dKr);
    return hipGetLastError();
}

}  // namespace

size_t route_bwd_workspace(int64_t B, int Tq, int Hq, int Hkv, int D, int64_t N, int64_t n_docs) {
    return rbwd_layout(B, Tq, Hq, Hkv, D, N, n_docs).total;
}

hipError_t launch_route_bwd(const RouteBwdArgs& a, hipStream_t st) {
    return a.r.dt == MSA_BF16 ? launch_rbwd_t<bf16_t>(a, st) : launch_rbwd_t<float>(a, st);
}

}  // namespace msa
