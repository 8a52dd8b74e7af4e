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
//                  U . k^ / Hq, in fp32 on the matrix cores) and, per chunk,
//                  the best token as one 64-bit key (score, then lowest token).
//   rbwd_docmax    per (b, doc) with a non-zero gradient: the best chunk key
//                  (lowest chunk among equal scores), then the per-head
//                  cosines at the arg max.
//   rbwd_dq        one workgroup per (b, t): the documents whose arg max token
//                  is t, in document order, summed into dQr[b, t].
//   rbwd_dk        one workgroup per document, one wave per chunk row: the
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

// |K̄r[n, g]| for every (chunk row, KV head): 16 lanes per row, 16 rows per
// workgroup.
template <typename T>
__global__ __launch_bounds__(256) void rbwd_knorm_kernel(const T* __restrict__ Kr, int64_t rows, int D,
                                                         float* __restrict__ knorm) {
    const int64_t row = int64_t(blockIdx.x) * 16 + threadIdx.x / 16;
    const int sub = threadIdx.x % 16;
    float s = 0.f;
    if (row < rows)
        for (int c = sub; c < D; c += 16) {
            const float x = Elem<T>::load(Kr, row * D + c);
            s += x * x;
        }
    s = group_sum<16>(s);
    if (row < rows && sub == 0) knorm[row] = sqrtf(s);
}

// Per chunk row n and query b: the best token, as the key
// order32(score) << 32 | (2^32 - 1 - t) (higher score, then lower t, wins).
// The scores U . k^ are a dense contraction (tokens x chunks over Hkv * D),
// run on the matrix cores in fp32 (v_mfma_f32_32x32x2_f32: fp32 products and
// sums, the precision of the vector path).  A workgroup takes 32 chunk rows
// and 256 tokens at a time, wave w the tokens 64w .. 64w+63 as two 32-row
// tiles; the contraction runs through LDS 32 elements at a time.  Two
// consecutive products take the elements e0 .. e0+3 with lane half u holding
// e0 + 2u and e0 + 2u + 1 (one 8-byte read per operand), the same pairing for
// both operands.
constexpr int kCB = 32;                       // chunk rows per workgroup
constexpr int kEB = 32;                       // contraction elements per LDS stage
constexpr int kSS = kEB + 2;                  // padded LDS row (conflict-free 8-byte reads)

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T>
__global__ __launch_bounds__(256) void rbwd_chunkmax_kernel(
    const float* __restrict__ U, int Tq, int Hq, const T* __restrict__ Kr, int64_t N, int hkv, int D,
    const float* __restrict__ knorm, unsigned long long* __restrict__ ckey) {
    __shared__ __attribute__((aligned(16))) float sU[256 * kSS];
    __shared__ __attribute__((aligned(16))) float sK[kCB * kSS];
    __shared__ unsigned long long s_key[4][kCB];
    const int64_t n0 = int64_t(blockIdx.x) * kCB;
    const int64_t b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid % kWave, half = lane / 32;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int RW = hkv * D;
    const int nb = int(N - n0 < kCB ? N - n0 : kCB);
    const float inv_hq = 1.f / float(Hq);
    unsigned long long best = 0ull;           // thread j < kCB: running best of chunk n0 + j
    for (int t0 = 0; t0 < Tq; t0 += 256) {
        f32x16 acc[2];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[m][i] = 0.f;
        for (int e0 = 0; e0 < RW; e0 += kEB) {
            __syncthreads();                   // every wave done with the previous stage
            for (int i = tid; i < 256 * (kEB / 4); i += 256) {
                const int r = i / (kEB / 4), c = (i % (kEB / 4)) * 4;
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (t0 + r < Tq) v = *reinterpret_cast<const float4*>(U + (b * Tq + t0 + r) * int64_t(RW) + e0 + c);
                *reinterpret_cast<float2*>(sU + r * kSS + c) = make_float2(v.x, v.y);
                *reinterpret_cast<float2*>(sU + r * kSS + c + 2) = make_float2(v.z, v.w);
            }
            for (int i = tid; i < kCB * kEB; i += 256) {
                const int j = i / kEB, c = i % kEB;
                float v = 0.f;
                if (j < nb) {
                    const int64_t n = n0 + j;
                    v = Elem<T>::load(Kr, n * RW + e0 + c) / fmaxf(knorm[n * hkv + (e0 + c) / D], kEps);
                }
                sK[j * kSS + c] = v;
            }
            __syncthreads();
#pragma unroll
            for (int c = 0; c < kEB; c += 4) {
                const float2 kb = *reinterpret_cast<const float2*>(sK + (lane % 32) * kSS + c + 2 * half);
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const float2 ua =
                        *reinterpret_cast<const float2*>(sU + (64 * wave + 32 * m + lane % 32) * kSS + c + 2 * half);
                    acc[m] = __builtin_amdgcn_mfma_f32_32x32x2f32(ua.x, kb.x, acc[m], 0, 0, 0);
                    acc[m] = __builtin_amdgcn_mfma_f32_32x32x2f32(ua.y, kb.y, acc[m], 0, 0, 0);
                }
            }
        }
        // best token of each chunk (the lane's column) over this block of tokens
        unsigned long long key = 0ull;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int t = t0 + 64 * wave + 32 * m + (i / 4) * 8 + half * 4 + (i % 4);
                if (t < Tq) {
                    const unsigned long long kk =
                        (static_cast<unsigned long long>(order32(acc[m][i] * inv_hq)) << 32) | (0xFFFFFFFFu - uint32_t(t));
                    key = kk > key ? kk : key;
                }
            }
        const unsigned long long other = __shfl_xor(key, 32);
        key = other > key ? other : key;
        if (lane < kCB) s_key[wave][lane] = key;
        __syncthreads();
        if (tid < kCB) {
#pragma unroll
            for (int w = 0; w < 4; ++w) best = s_key[w][tid] > best ? s_key[w][tid] : best;
        }
    }
    if (tid < nb) ckey[b * N + n0 + tid] = best;
}

// Per (b, doc) with a non-zero gradient: the arg max over the document's
// chunks (the first chunk among equal scores) of the per-chunk best keys,
// then the per-head cosines there.
template <typename T>
__global__ __launch_bounds__(256) void rbwd_docmax_kernel(
    const T* __restrict__ Qr, int Tq, int Hq, const T* __restrict__ Kr, int64_t N, int hkv, int D,
    const int64_t* __restrict__ chunk_off, int64_t n_docs, const float* __restrict__ dscore,
    const unsigned long long* __restrict__ ckey, const float* __restrict__ knorm, int2* __restrict__ arg,
    float* __restrict__ cosv) {
    const int64_t doc = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int64_t bd = b * n_docs + doc;
    int64_t n_lo = chunk_off[doc], n_hi = chunk_off[doc + 1];
    n_lo = n_lo < 0 ? 0 : (n_lo > N ? N : n_lo);
    n_hi = n_hi < n_lo ? n_lo : (n_hi > N ? N : n_hi);
    if (dscore[bd] == 0.f || n_hi == n_lo) {
        if (threadIdx.x == 0) arg[bd] = make_int2(-1, -1);
        return;
    }
    // lane-strided scan, then a wave max of (score, -chunk, -token) (every wave
    // finds the same arg max)
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
    if (threadIdx.x == 0) arg[bd] = make_int2(int(n), t);
    const int G = Hq / hkv;
    for (int h = wave; h < Hq; h += 4) {
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

// One workgroup per document, one wave per chunk row of it (waves stride
// the rows): the queries whose arg max chunk is the row, in query order.
template <typename T>
__global__ __launch_bounds__(256) void rbwd_dk_kernel(
    const T* __restrict__ Kr, int64_t N, int hkv, int D, int Tq, int Hq, const int64_t* __restrict__ chunk_off,
    int64_t n_docs, int64_t B, const float* __restrict__ dscore, const float* __restrict__ U,
    const float* __restrict__ knorm, const int2* __restrict__ arg, const float* __restrict__ cosv,
    float* __restrict__ dKr) {
    const int64_t doc = blockIdx.x;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    int64_t n_lo = chunk_off[doc], n_hi = chunk_off[doc + 1];
    n_lo = n_lo < 0 ? 0 : (n_lo > N ? N : n_lo);
    n_hi = n_hi < n_lo ? n_lo : (n_hi > N ? N : n_hi);
    const int RW = hkv * D;
    const int G = Hq / hkv;
    const float inv_hq = 1.f / float(Hq);
    constexpr int kMaxPer = 32;                // elements per lane: RW <= 2048
    const int per = RW / kWave;
    for (int64_t n = n_lo + wave; n < n_hi; n += 4) {
        float acc[kMaxPer];
#pragma unroll
        for (int i = 0; i < kMaxPer; ++i) acc[i] = 0.f;
        bool any = false;
        for (int64_t b = 0; b < B; ++b) {
            const int2 a = arg[b * n_docs + doc];
            if (a.x != int(n)) continue;
            any = true;
            const float w = dscore[b * n_docs + doc] * inv_hq;
            const float* ur = U + (b * Tq + a.y) * int64_t(RW);
#pragma unroll
            for (int i = 0; i < kMaxPer; ++i)
                if (i < per) acc[i] += w * ur[lane + kWave * i];
        }
        if (!any) {                            // no gradient reaches this row
#pragma unroll
            for (int i = 0; i < kMaxPer; ++i)
                if (i < per) dKr[n * RW + lane + kWave * i] = 0.f;
            continue;
        }
#pragma unroll
        for (int i = 0; i < kMaxPer; ++i) {
            if (i >= per) break;
            const int e = lane + kWave * i, g = e / D;
            // the same queries' w sum_{h in g} c_h
            float c = 0.f;
            for (int64_t b = 0; b < B; ++b) {
                const int2 a = arg[b * n_docs + doc];
                if (a.x != int(n)) continue;
                float cs = 0.f;
                for (int h = g * G; h < (g + 1) * G; ++h) cs += cosv[(b * n_docs + doc) * Hq + h];
                c += dscore[b * n_docs + doc] * inv_hq * cs;
            }
            const float nk = knorm[n * hkv + g];
            float d;
            if (nk > kEps) d = (acc[i] - c * Elem<T>::load(Kr, n * RW + e) / nk) / nk;
            else d = acc[i] / kEps;
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
    hipLaunchKernelGGL((rbwd_knorm_kernel<T>), dim3(unsigned(ceil_div(r.N * r.Hkv, int64_t(16)))), dim3(256), 0, st,
                       Kr, r.N * r.Hkv, r.D, knorm);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((rbwd_chunkmax_kernel<T>), dim3(unsigned(ceil_div(r.N, int64_t(kCB))), unsigned(r.B)),
                       dim3(256), 0, st, U, r.Tq, r.Hq, Kr, r.N, r.Hkv, r.D, knorm, ckey);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((rbwd_docmax_kernel<T>), dim3(unsigned(r.n_docs), unsigned(r.B)), dim3(256), 0, st, Qr, r.Tq,
                       r.Hq, Kr, r.N, r.Hkv, r.D, r.chunk_off, r.n_docs, a.dscore, ckey, knorm, arg, cosv);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const size_t dq_lds = size_t(r.Hkv * r.D + 2 * r.Hq) * sizeof(float);
    hipLaunchKernelGGL((rbwd_dq_kernel<T>), dim3(unsigned(r.Tq), unsigned(r.B)), dim3(256), dq_lds, st, Qr, r.Tq,
                       r.Hq, Kr, r.Hkv, r.D, r.n_docs, a.dscore, knorm, arg, cosv, a.dQr);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((rbwd_dk_kernel<T>), dim3(unsigned(r.n_docs)), dim3(256), 0, st, Kr, r.N,
                       r.Hkv, r.D, r.Tq, r.Hq, r.chunk_off, r.n_docs, r.B, a.dscore, U, knorm, arg, cosv, a.dKr);
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
