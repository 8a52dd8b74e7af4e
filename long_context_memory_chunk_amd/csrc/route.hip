// Stage 2a (online): cosine routing score, per-document max, top-k.
//
// Source: news.neo-ai.one MSA article, 全体設計 › アーキテクチャ (Fig. 2):
// relevance is the cosine similarity of Qr with K̄r, averaged over heads and
// then maximised over tokens, and the top-k documents are selected;
// 推論パイプライン (Fig. 3): K̄r is matched online.  ruixiangma.github.io blog,
// 方法 › 稀疏注意力机制 (top-k documents by cosine).  github-eval-reports
// review, 核心模块 (head mean first, then token max).
//
// Order of the call: route_prep (U, the unit-query group sums; skipped where
// the scan forms U itself), then the chunk scores c[B][N] from one of three scans -- the VALU streaming scan or
// the generic one (route_scan.hip), or the matrix-core path (route_mfma.hip)
// -- then the two top-k kernels below.
//
// Kernels
//   topk_partial          per-wave document max (LDS segmented max over
//                         coalesced chunk-score loads): every document's key
//                         bits and each wave's largest key.
//   topk_final            the K-th largest wave maximum bounds the K-th key
//                         from below, and the wave maxima are distinct keys,
//                         so at most K waves reach it; their documents are
//                         read in one batched pass and the top k of the keys
//                         at or above the bound kept.
// (A single kernel whose last workgroup does the final step was measured
// slower: the device-scope fences that publish every workgroup's results
// cost more than the second launch.)
// The top-k key is 64 bits: order-preserving bits of the fp32 document
// score above (0xFFFFFFFF - doc id), so a larger key is a better document
// and equal scores order by lower id, a total order.
#include "common.hpp"
#include "launch.hpp"
#include "route_mfma.hpp"
#include "route_scan.hpp"

namespace msa {
namespace {

// ---------------------------------------------------------------- top-k

__device__ __forceinline__ uint64_t make_key(float s, uint32_t id) {
    s = s + 0.0f;                                   // -0 -> +0
    const uint32_t u = __float_as_uint(s);
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (uint64_t(o) << 32) | uint64_t(0xFFFFFFFFu - id);
}

__device__ __forceinline__ float key_score(uint64_t k) {
    const uint32_t o = uint32_t(k >> 32);
    const uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
    const uint32_t lo = uint32_t(__shfl_xor(int(uint32_t(v)), m));
    const uint32_t hi = uint32_t(__shfl_xor(int(uint32_t(v >> 32)), m));
    return (uint64_t(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t shfl64(uint64_t v, int src) {
    const uint32_t lo = uint32_t(__shfl(int(uint32_t(v)), src));
    const uint32_t hi = uint32_t(__shfl(int(uint32_t(v >> 32)), src));
    return (uint64_t(hi) << 32) | lo;
}

// Bitonic sort of one key per lane, descending across lanes 0..63.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t x, int lane) {
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint64_t y = shfl_xor64(x, j);
            const bool desc_block = (lane & k) == 0;
            const bool lower = (lane & j) == 0;
            const uint64_t mx = x > y ? x : y, mn = x > y ? y : x;
            x = (lower == desc_block) ? mx : mn;
        }
    }
    return x;
}

// best and x sorted descending across lanes; returns the top 64 of both.
__device__ __forceinline__ uint64_t wave_merge_desc(uint64_t best, uint64_t x, int lane) {
    const uint64_t xr = shfl64(x, 63 - lane);
    uint64_t c = best > xr ? best : xr;             // bitonic
#pragma unroll
    for (int j = 32; j > 0; j >>= 1) {
        const uint64_t y = shfl_xor64(c, j);
        const bool lower = (lane & j) == 0;
        const uint64_t mx = c > y ? c : y, mn = c > y ? y : c;
        c = lower ? mx : mn;
    }
    return c;
}

// Offers one key per lane to the running top-K list `best` (sorted
// descending across lanes, distinct keys, zeros as padding).  A few winners
// are inserted one at a time (one ballot and two shuffles each); many are
// sorted and merged.
__device__ __forceinline__ uint64_t wave_offer(uint64_t best, uint64_t key, int K, int lane) {
    const uint64_t kth = shfl64(best, K - 1);
    uint64_t mask = __ballot(key > kth);
    if (mask == 0) return best;
    if (__popcll(mask) > 8) return wave_merge_desc(best, wave_sort_desc(key, lane), lane);
    while (mask) {
        const int src = __ffsll((unsigned long long)mask) - 1;
        mask &= mask - 1;
        const uint64_t x = shfl64(key, src);
        if (x <= shfl64(best, K - 1)) continue;          // beaten by an earlier insertion
        const int pos = __popcll(__ballot(best > x));
        const uint64_t prev = shfl64(best, lane > 0 ? lane - 1 : 0);
        best = (lane < pos) ? best : (lane == pos ? x : prev);
    }
    return best;
}

__device__ __forceinline__ uint32_t order32(float s) {
    s = s + 0.0f;                                   // -0 -> +0
    const uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unorder32(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Wave w of query b owns documents [S w, S w + S), S = kDocsPerWave (128, or
// 512 for banks of many documents, see topk_docs_per_wave).  It stages their
// chunk offsets in LDS, streams the chunk scores of their span with
// coalesced loads, finds each chunk's document and takes an LDS atomic max on
// the order-preserving bits (max is exact and order-independent, so the result
// is deterministic), then writes every document's bits and the wave's largest
// composite key.
// A chunk's document: the wave marks each document's first chunk as a bit in
// LDS; for a window of 64 chunks, the lane's document is the number of marks
// at or before its chunk (a popcount of the window's 64-bit mask under the
// lane mask, plus the marks of earlier windows) minus one.  A wave whose span
// exceeds the bit array, or that holds an empty document (two documents would
// share one mark), finds documents by binary search in the offsets instead.
constexpr int kBitWords = 1024;                  // marks for spans of up to 32768 chunks per wave

template <int kDocsPerWave>
__global__ __launch_bounds__(256) void topk_partial_kernel(
    const float* __restrict__ c, int64_t N, const int64_t* __restrict__ off, int64_t n_docs,
    int waves_per_b, uint32_t* __restrict__ dkey, uint64_t* __restrict__ wmax, float* __restrict__ out_doc) {
    __shared__ int64_t s_off[4][kDocsPerWave + 1];
    __shared__ uint32_t s_max[4][kDocsPerWave];
    __shared__ uint32_t s_bits[4][kBitWords + 2];
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    const int w = blockIdx.x * 4 + wv;
    const bool active = w < waves_per_b;
    const int64_t b = blockIdx.y;
    const int64_t d0 = int64_t(w) * kDocsPerWave;
    int nd = 0;
    if (active) {
        const int64_t rem = n_docs - d0;
        nd = int(rem < kDocsPerWave ? rem : kDocsPerWave);
    }
    for (int j = lane; j <= kDocsPerWave; j += kWave) {
        int64_t o = 0;
        if (j <= nd) {
            o = off[d0 + j];
            o = o < 0 ? 0 : (o > N ? N : o);
        }
        s_off[wv][j] = o;
    }
    for (int j = lane; j < kDocsPerWave; j += kWave) s_max[wv][j] = 0u;
    __syncthreads();

    const int64_t lo_bound = s_off[wv][0];
    const int64_t c1 = s_off[wv][nd];
    const int64_t span = c1 - lo_bound;
    bool ok = span <= int64_t(kBitWords) * 32;
    for (int j = lane; j < nd; j += kWave) ok = ok && (s_off[wv][j + 1] > s_off[wv][j]);
    const bool marks = nd > 0 && __all(ok);
    if (marks) {
        const int words = int((span + 31) / 32) + 2;
        for (int i = lane; i < words; i += kWave) s_bits[wv][i] = 0u;
    }
    __syncthreads();
    if (marks) {
        for (int j = lane; j < nd; j += kWave) {
            const int t = int(s_off[wv][j] - lo_bound);
            atomicOr(&s_bits[wv][t >> 5], 1u << (t & 31));
        }
    }
    __syncthreads();

    if (nd > 0) {
        const float* cb = c + b * N;
        if (marks) {
            const uint64_t le = (lane == 63) ? ~0ull : ((1ull << (lane + 1)) - 1);
            int before = 0;                          // marks in earlier windows
            constexpr int U = 32;                    // windows whose loads are in flight together
            for (int64_t n0 = lo_bound; n0 < c1; n0 += kWave * U) {
                float v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t n = n0 + u * kWave + lane;
                    v[u] = (n < c1) ? cb[n] : 0.f;
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t w0 = n0 + u * kWave;
                    if (w0 >= c1) break;
                    const int t0 = int(w0 - lo_bound);   // multiple of 64: the window is words t0/32, t0/32 + 1
                    const uint64_t m = uint64_t(s_bits[wv][t0 >> 5]) | (uint64_t(s_bits[wv][(t0 >> 5) + 1]) << 32);
                    const int doc = before + __popcll(m & le) - 1;
                    before += __popcll(m);
                    if (w0 + lane < c1) atomicMax(&s_max[wv][doc], order32(v[u]));
                }
            }
        } else {
            for (int64_t n0 = lo_bound; n0 < c1; n0 += kWave) {
                const int64_t n = n0 + lane;
                if (n < c1) {
                    const float v = cb[n];
                    int lo = 0, hi = nd;                 // largest j with s_off[j] <= n
                    while (hi - lo > 1) {
                        const int mid = (lo + hi) >> 1;
                        if (s_off[wv][mid] <= n) lo = mid; else hi = mid;
                    }
                    atomicMax(&s_max[wv][lo], order32(v));
                }
            }
        }
    }
    __syncthreads();
    // each document's order-preserving score bits (0: no chunks), and the
    // largest composite key (score, then lowest id) of the wave
    uint64_t wbest = 0;
    for (int j = lane; j < nd; j += kWave) {
        const bool has = s_off[wv][j + 1] > s_off[wv][j];
        const uint32_t o = has ? s_max[wv][j] : 0u;
        if (out_doc && has) out_doc[b * n_docs + d0 + j] = unorder32(o);
        dkey[b * n_docs + d0 + j] = o;
        const uint64_t key = has ? ((uint64_t(o) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(d0 + j))) : 0;
        wbest = key > wbest ? key : wbest;
    }
#pragma unroll
    for (int j = 32; j > 0; j >>= 1) {
        const uint64_t y = shfl_xor64(wbest, j);
        wbest = y > wbest ? y : wbest;
    }
    if (active && lane == 0) wmax[b * waves_per_b + w] = wbest;
}

// One workgroup per query.  The K largest wave maxima are K distinct
// documents, so the K-th of them (thr) is at most the K-th largest key
// overall: every top-K document has a key >= thr and lies in a wave whose
// maximum is >= thr, and only K waves have one (the maxima are distinct).
// (a) The wave maxima are loaded once (kept in LDS when they fit); 16 waves
// reduce them to their top K and a pairwise merge tree combines the 16 lists
// (thr); (b) the waves that reach thr are listed; (c) every thread reads its
// share of those waves' document keys in one batch of loads and keeps the
// keys >= thr in LDS; (d) wave 0 offers those to its top K.  If ties make
// more keys qualify than the buffer holds, wave 0 offers every document of
// the qualifying waves instead (exact, slower).
constexpr int kFinalWaves = 16;
constexpr int kFinalThreads = kFinalWaves * 64;
constexpr int kSelCap = 4096;
constexpr int kWmaxLds = 4096;                   // wave maxima kept in LDS (larger banks re-read them)

template <int kDocsPerWave>
__global__ __launch_bounds__(kFinalThreads) void topk_final_kernel(
    const uint32_t* __restrict__ dkey, int64_t n_docs, const uint64_t* __restrict__ wmax, int W, int K,
    int32_t* __restrict__ ids, float* __restrict__ scores) {
    __shared__ uint64_t lists[kFinalWaves][64];
    __shared__ uint64_t sel[kSelCap];
    __shared__ uint64_t s_wm[kWmaxLds];
    __shared__ int qual[MSA_MAX_TOPK];
    __shared__ int s_count, s_nq;
    __shared__ uint64_t s_thr;
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int64_t b = blockIdx.x;
    const uint64_t* wm = wmax + b * W;
    const uint32_t* db = dkey + b * n_docs;
    const bool wm_lds = W <= kWmaxLds;
    constexpr int kDocsPerThread = MSA_MAX_TOPK * kDocsPerWave / kFinalThreads;

    // (a) thr = the K-th largest wave maximum
    const int per = ((W + kFinalWaves - 1) / kFinalWaves + kWave - 1) / kWave * kWave;
    const int c0 = wave * per, c1 = (c0 + per < W) ? c0 + per : W;
    uint64_t best = 0;
    for (int base = c0; base < c1; base += kWave) {
        const uint64_t m = (base + lane < c1) ? wm[base + lane] : 0;
        if (wm_lds && base + lane < c1) s_wm[base + lane] = m;
        best = wave_offer(best, m, K, lane);
    }
    lists[wave][lane] = (lane < K) ? best : 0;
    if (tid == 0) { s_count = 0; s_nq = 0; }
    __syncthreads();
    // pairwise merge tree of the 16 sorted lists (4 levels)
#pragma unroll
    for (int active = kFinalWaves / 2; active >= 1; active >>= 1) {
        uint64_t m = 0;
        if (wave < active) m = wave_merge_desc(lists[2 * wave][lane], lists[2 * wave + 1][lane], lane);
        __syncthreads();
        if (wave < active) lists[wave][lane] = (lane < K) ? m : 0;
        __syncthreads();
    }
    if (tid == 0) s_thr = lists[0][K - 1];
    __syncthreads();
    const uint64_t thr = s_thr;

    // (b) the waves that reach thr: at most K
    for (int i = tid; i < W; i += kFinalThreads) {
        const uint64_t m = wm_lds ? s_wm[i] : wm[i];
        if (m != 0 && m >= thr) {
            const int p = atomicAdd(&s_nq, 1);
            if (p < MSA_MAX_TOPK) qual[p] = i;
        }
    }
    __syncthreads();
    const int nq = s_nq < MSA_MAX_TOPK ? s_nq : MSA_MAX_TOPK;

    // (c) their document keys, one batch of loads per thread: entry e of the
    // nq * 128 documents is thread e % 1024's load e / 1024
    {
        uint32_t o[kDocsPerThread];
#pragma unroll
        for (int u = 0; u < kDocsPerThread; ++u) {
            const int e = u * kFinalThreads + tid;
            int64_t doc = n_docs;
            if (e < nq * kDocsPerWave) doc = int64_t(qual[e / kDocsPerWave]) * kDocsPerWave + e % kDocsPerWave;
            o[u] = doc < n_docs ? db[doc] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kDocsPerThread; ++u) {
            const int e = u * kFinalThreads + tid;
            if (o[u] == 0u || e >= nq * kDocsPerWave) continue;
            const int64_t doc = int64_t(qual[e / kDocsPerWave]) * kDocsPerWave + e % kDocsPerWave;
            const uint64_t key = (uint64_t(o[u]) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(doc));
            if (key >= thr) {
                const int p = atomicAdd(&s_count, 1);
                if (p < kSelCap) sel[p] = key;
            }
        }
    }
    __syncthreads();
    const int count = s_count;
    if (wave != 0) return;

    // (d) the top K
    best = 0;
    if (count <= kSelCap) {
        for (int base = 0; base < count; base += kWave)
            best = wave_offer(best, (base + lane < count) ? sel[base + lane] : 0, K, lane);
    } else {
        for (int q = 0; q < nq; ++q)
            for (int j0 = 0; j0 < kDocsPerWave; j0 += kWave) {
                const int64_t doc = int64_t(qual[q]) * kDocsPerWave + j0 + lane;
                uint64_t key = 0;
                if (doc < n_docs) {
                    const uint32_t o = db[doc];
                    if (o != 0) key = (uint64_t(o) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(doc));
                }
                best = wave_offer(best, key, K, lane);
            }
    }
    if (lane < K) {
        ids[b * K + lane] = int32_t(0xFFFFFFFFu - uint32_t(best));
        if (scores) scores[b * K + lane] = key_score(best);
    }
}

// Documents per wave of topk_partial: 128 (the measured best on the 100M-token
// bank's 199,922 documents: 21.5 us for the two kernels, against 24.4 with
// 256 and 23.7 with 64), or 512 when 128 would give topk_final more wave
// maxima than it keeps in LDS (chunk-level selection: 1,562,500 candidates).
int topk_docs_per_wave(int64_t n_docs) {
    return ceil_div(n_docs, int64_t(128)) <= kWmaxLds ? 128 : 512;
}

int topk_waves(int64_t n_docs, int dpw) {
    const int64_t w = ceil_div(n_docs, int64_t(dpw));
    return int(w < 1 ? 1 : w);
}

struct RouteWs {
    size_t u_off, c_off, dkey_off, wmax_off, mfma_off, total;
};

RouteWs route_ws_layout(msa_dtype dt, int64_t B, int Tq, int Hq, int Hkv, int D, int64_t N,
                        int64_t n_docs, int top_k, int num_cus) {
    RouteWs w;
    const int64_t nq = B * Tq;
    size_t o = 0;
    w.u_off = o;   o += align256(size_t(nq) * Hkv * D * sizeof(float));
    w.c_off = o;   o += align256(size_t(B) * N * sizeof(float));
    w.dkey_off = o; o += align256(size_t(B) * n_docs * sizeof(uint32_t));
    w.wmax_off = o; o += align256(size_t(B) * topk_waves(n_docs, topk_docs_per_wave(n_docs)) * sizeof(uint64_t));
    w.mfma_off = o; o += align256(route_mfma_workspace(dt, B, Tq, Hq, Hkv, D, N, num_cus));
    w.total = o;
    return w;
}

}  // namespace

size_t route_workspace(msa_dtype dt, int64_t B, int Tq, int Hq, int Hkv, int D, int64_t N,
                       int64_t n_docs, int top_k, int num_cus) {
    return route_ws_layout(dt, B, Tq, Hq, Hkv, D, N, n_docs, top_k, num_cus).total;
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
    const RouteWs w = route_ws_layout(a.dt, a.B, a.Tq, a.Hq, a.Hkv, a.D, a.N, a.n_docs, a.top_k,
                                      a.num_cus);
    char* ws = static_cast<char*>(a.ws);
    float* U = reinterpret_cast<float*>(ws + w.u_off);
    float* c = a.out_chunk ? a.out_chunk : reinterpret_cast<float*>(ws + w.c_off);
    uint32_t* dkey = reinterpret_cast<uint32_t*>(ws + w.dkey_off);
    uint64_t* wmax = reinterpret_cast<uint64_t*>(ws + w.wmax_off);
    hipError_t err;

    // 1. unit-query group sums (the streaming scan with an aligned query, and
    // the matrix-core path of decode batches and short queries, form them
    // themselves; the latter in its bf16 operand layout)
    const bool preps_itself = a.N > 0 && (route_scan_fast_applicable(a) ? route_scan_fast_preps_itself(a)
                                                                         : route_mfma_preps_itself(a));
    if (!preps_itself)
        if ((err = launch_route_prep(a, U, st)) != hipSuccess) return err;

    // 2. chunk scores c[B][N]; the chunk-score kernel's dispatch records the
    // profiling events itself (an empty bank records them back to back)
    if (a.N == 0) {
        if ((err = record_if(a.prof_start, st)) != hipSuccess) return err;
        if ((err = record_if(a.prof_stop, st)) != hipSuccess) return err;
    } else if (route_scan_fast_applicable(a)) {
        if ((err = launch_route_scan_fast(a, U, c, st)) != hipSuccess) return err;
    } else if (route_mfma_applicable(a.dt, a.B, a.Tq, a.Hkv, a.D)) {
        if ((err = launch_route_mfma(a, U, c, ws + w.mfma_off, st)) != hipSuccess) return err;
    } else {
        if ((err = launch_route_scan_generic(a, U, c, st)) != hipSuccess) return err;
    }

    // 3. document max + top-k
    const int dpw = topk_docs_per_wave(a.n_docs);
    const int wpb = topk_waves(a.n_docs, dpw);
#define MSA_TOPK(S)                                                                                           \
    hipLaunchKernelGGL(topk_partial_kernel<S>, dim3(unsigned(ceil_div(wpb, 4)), unsigned(a.B)), dim3(256), 0, \
                       st, c, a.N, a.chunk_off, a.n_docs, wpb, dkey, wmax, a.out_doc);                      \
    if ((err = hipGetLastError()) != hipSuccess) return err;                                                 \
    hipLaunchKernelGGL(topk_final_kernel<S>, dim3(unsigned(a.B)), dim3(kFinalThreads), 0, st, dkey,         \
                       a.n_docs, wmax, wpb, a.top_k, a.out_ids, a.out_scores);
    if (dpw == 128) {
        MSA_TOPK(128)
    } else {
        MSA_TOPK(512)
    }
#undef MSA_TOPK
    return hipGetLastError();
}

}  // namespace msa
