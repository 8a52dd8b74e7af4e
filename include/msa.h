/*
 * msa.h -- C ABI of the Memory Sparse Attention (MSA) hot path on one
 * AMD Instinct MI355X (gfx950).
 *
 * MSA is described on these pages:
 *   [neo]   news.neo-ai.one MSA article: 全体設計 › アーキテクチャ (Fig. 2),
 *           推論パイプライン (Fig. 3)
 *   [blog]  ruixiangma.github.io "Memory-Sparse-Attention": 方法 ›
 *           稀疏注意力机制, 文档级RoPE, 三阶段推理流程, Memory Parallel
 *   [aip]   ai-papers.net MSA summary: MSAの提案手法
 *   [rev]   github-eval-reports review of MSA: 推理流程, 核心模块
 *
 * The calls follow the three-stage pipeline of [neo] 推論パイプライン and
 * [blog] 三阶段推理流程:
 *   1. offline global memory encoding  -> msa_encode_pool
 *   2. online routing + context build  -> msa_route, msa_gather
 *   3. sparse generation               -> msa_sparse_attn
 *
 * Conventions for every call
 *   - All tensors are row-major and densely packed.  "device" pointers are
 *     HIP device memory on the context's device; "host" pointers are CPU
 *     memory.  bf16 tensors hold raw bfloat16 bit patterns (uint16).
 *   - The caller allocates and owns every buffer and every stream; the
 *     library allocates only the context's RoPE table.  Workspaces are
 *     caller-provided device buffers of at least the size the matching
 *     *_workspace_size() call returns, aligned to 256 bytes.
 *   - Calls are asynchronous on the given stream unless stated otherwise.
 *     Arguments are validated synchronously, before anything is enqueued;
 *     on any error nothing is enqueued.  Launch failures map to
 *     MSA_ERR_HIP.  Faults inside a kernel surface at the caller's next
 *     synchronisation.  No C++ exception crosses the ABI.
 *   - msa_last_error() returns a message for the last failing call on the
 *     calling thread (thread-local; valid until that thread's next call).
 *   - Inputs are assumed finite (no NaN/Inf); this is not checked.
 *   - Head dim d is 64 or 128 (fixed per context); Hq % Hkv == 0.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_ABI_VERSION 2
#define MSA_MAX_TOPK 64

typedef enum msa_status {
    MSA_OK = 0,
    MSA_ERR_INVALID_ARG = 1,  /* a pointer, size or relation is wrong      */
    MSA_ERR_UNSUPPORTED = 2,  /* valid request this build does not handle  */
    MSA_ERR_HIP = 3,          /* a HIP runtime call or launch failed       */
    MSA_ERR_WORKSPACE = 4     /* workspace null, misaligned or too small   */
} msa_status;

typedef enum msa_dtype {
    MSA_F32 = 0,              /* IEEE binary32                             */
    MSA_BF16 = 1              /* bfloat16 bits; fp32 accumulation inside   */
} msa_dtype;

typedef struct msa_ctx msa_ctx;

/* ABI version compiled into the library (MSA_ABI_VERSION). */
int msa_abi_version(void);

/* Message of the last failing call on this thread ("" if none). */
const char* msa_last_error(void);

/* Static name of a status code. */
const char* msa_status_string(msa_status s);

/*
 * msa_ctx_create -- bind the library to `device` and build the RoPE table.
 *
 * Rotary embedding in rotate-half form ([neo] アーキテクチャ: parallel /
 * document-wise RoPE and global RoPE; the pages give no formula, the
 * backbone's rotate-half form is used): element i pairs with i + d/2,
 * angle(pos, i) = pos * rope_theta^(-2i/d).  The table cos/sin[max_pos][d/2]
 * is computed on the host from float64 angles and stored as float32 on the
 * device (owned by the context, freed by msa_ctx_destroy).  Every position a
 * later call uses (document-local token index, top_k + local index) must be
 * < max_pos.  Synchronous.
 *   device     HIP device ordinal; must be a gfx950 device.
 *   head_dim   64 or 128.
 *   rope_theta > 1.
 *   max_pos    1 .. 1<<22.
 *   out        receives the context; untouched on error.
 */
msa_status msa_ctx_create(int device, int head_dim, double rope_theta, int max_pos,
                          msa_ctx** out);

/* Frees the context and its table.  Synchronises the device first.  NULL ok. */
msa_status msa_ctx_destroy(msa_ctx* ctx);

/*
 * msa_chunk_offsets -- host helper, synchronous.  Chunk-row layout of a
 * pooled bank ([neo] アーキテクチャ, [blog] 稀疏注意力机制: every document is
 * split into fixed-length chunks): document d has ceil(len_d / chunk_len)
 * chunks, stored at rows doc_chunk_off[d] .. doc_chunk_off[d+1]-1.
 *   doc_tok_off      host int64[n_docs+1], doc_tok_off[0] == 0, strictly
 *                    increasing (every document has >= 1 token).
 *   doc_chunk_off    host int64[n_docs+1] output.
 *   max_doc_len      host output or NULL: the longest document's length in
 *                    tokens (0 when n_docs == 0), the value msa_encode_pool
 *                    and msa_encode_pool_bwd take as max_doc_len.
 */
msa_status msa_chunk_offsets(const int64_t* doc_tok_off, int64_t n_docs, int chunk_len,
                             int64_t* doc_chunk_off, int64_t* max_doc_len);

/*
 * msa_encode_pool -- stage 1 (offline): document-wise RoPE + chunk mean.
 * ([neo] アーキテクチャ and 推論パイプライン first stage; [blog] 稀疏注意力机制,
 * 文档级RoPE; [aip] MSAの提案手法.)
 * For document d with tokens [s, e) and its chunk j covering rows
 * r in [s + j*c, min(s + (j+1)*c, e)):
 *     K̄  = mean_r RoPE(K[r], r - s)     (positions restart at 0 per document)
 *     V̄  = mean_r V[r]
 *     K̄r = mean_r Kr[r]
 * summed in fp32, divided by the actual row count, rounded once to `dt`.
 *   K, V, Kr       device [T][Hkv][d] of dt, unrotated.
 *   doc_tok_off    device int64[n_docs+1] token offsets (as for
 *                  msa_chunk_offsets).
 *   doc_chunk_off  device int64[n_docs+1], the msa_chunk_offsets result.
 *   N              number of chunk rows = doc_chunk_off[n_docs].
 *   KVbar          device [N][2][Hkv][d] of dt: row n holds K̄ then V̄, so a
 *                  document's pooled content is one contiguous span.
 *   Krbar          device [N][Hkv][d] of dt.
 *   max_doc_len    host: the longest document's length in tokens (from
 *                  msa_chunk_offsets).  Document-local positions run up to
 *                  max_doc_len - 1, so max_doc_len > the context's max_pos
 *                  is MSA_ERR_INVALID_ARG, nothing enqueued.
 * Offsets are trusted to be consistent (use msa_chunk_offsets); if they are
 * not, outputs are unspecified but every access stays inside [0, T) rows
 * and [0, N) chunk rows.  A document that the device offsets make longer
 * than max_doc_len (a wrong max_doc_len) gets NaN in all of its pooled
 * rows: positions are never clamped or read past the RoPE table.
 */
msa_status msa_encode_pool(msa_ctx* ctx, msa_dtype dt,
                           const void* K, const void* V, const void* Kr,
                           const int64_t* doc_tok_off, const int64_t* doc_chunk_off,
                           int64_t n_docs, int64_t T, int64_t N, int Hkv, int chunk_len,
                           int64_t max_doc_len, void* KVbar, void* Krbar, hipStream_t stream);

/*
 * msa_encode_pool_bwd -- gradients of msa_encode_pool with respect to the
 * document tokens' K, V and Kr, given the gradients of the pooled rows.
 * (Training: [neo] アーキテクチャ pools each document's K/V/Kr by chunk means
 * with document-wise RoPE; [rev] 核心能力 › 端到端可训练框架: the memory is
 * trained end to end, so the gradients of the pooled rows reach the tokens.)
 * For document d with tokens [s, e) and its chunk j of rows [r0, r1):
 *     dK[r]  = RoPE^-1(dK̄[j] / (r1 - r0), r - s)   (rotation back by -angle)
 *     dV[r]  = dV̄[j] / (r1 - r0)
 *     dKr[r] = dK̄r[j] / (r1 - r0)
 *   dKVbar         device [N][2][Hkv][d] of dt (dK̄ then dV̄ per row, the
 *                  layout of msa_encode_pool's KVbar).
 *   dKrbar         device [N][Hkv][d] of dt.
 *   doc_tok_off, doc_chunk_off, n_docs, T, N, Hkv, chunk_len, max_doc_len
 *                  as for msa_encode_pool (the same checks; token rows of a
 *                  document longer than max_doc_len get NaN).
 *   dK, dV, dKr    device [T][Hkv][d] of dt (written for every token of a
 *                  document; rows outside every document untouched).
 * fp32 arithmetic, one rounding to dt on store.
 */
msa_status msa_encode_pool_bwd(msa_ctx* ctx, msa_dtype dt,
                               const void* dKVbar, const void* dKrbar,
                               const int64_t* doc_tok_off, const int64_t* doc_chunk_off,
                               int64_t n_docs, int64_t T, int64_t N, int Hkv, int chunk_len,
                               int64_t max_doc_len, void* dK, void* dV, void* dKr, hipStream_t stream);

/*
 * msa_route -- stage 2a (online): cosine routing + document top-k.
 * ([neo] アーキテクチャ: cosine similarity, mean over heads, then max over
 * tokens, top-k documents; [blog] 稀疏注意力机制; [rev] 核心模块.)
 * B independent queries of Tq tokens each; one pass over Krbar serves all.
 *     cos(q, k) = q.k / (max(|q|, 1e-8) * max(|k|, 1e-8))
 *     s[b,t,n]  = (1/Hq) sum_h cos(Qr[b,t,h], Krbar[n, h / (Hq/Hkv)])
 *     c[b,n]    = max_t s[b,t,n]                       (chunk score)
 *     D[b,doc]  = max over the document's chunk rows of c[b,n]
 *     out_ids[b] = the top_k documents by (D descending, id ascending),
 *                  in that order (ties go to the lowest id).
 *   Qr             device [B][Tq][Hq][d] of dt.
 *   Krbar          device [N][Hkv][d] of dt, resident in HBM.
 *   doc_chunk_off  device int64[n_docs+1], every document >= 1 chunk,
 *                  doc_chunk_off[n_docs] == N (trusted; accesses clamped).
 *   top_k          1 .. min(n_docs, MSA_MAX_TOPK).
 *   out_ids        int32[B][top_k], device memory or pinned host memory
 *                  (hipHostMalloc): a pinned buffer lets the host read the
 *                  ids right after the stream reaches the end of the call.
 *   out_scores     device float[B][top_k] (D of each selected id), or NULL.
 *   out_chunk      device float[B][N] receives c, or NULL (then c lives in
 *                  the workspace).
 *   out_doc        device float[B][n_docs] receives D, or NULL.
 *   workspace      device, >= msa_route_workspace_size(...) bytes.
 * bf16 routing at d = 128 with B*Tq > 4 contracts on the matrix cores (a
 * query of any length is padded to whole row tiles whose padding is left out
 * of the token max), with the head-group sum of the unit query vectors
 * rounded to bf16 (relative error <= 2^-9 per element, so a score moves by at
 * most 2^-9); a query of at least 1,024 tokens, or a multiple of 256, takes
 * one GEMM that also rounds the unit keys to bf16 (at most 2^-8).  Other
 * cases accumulate in fp32 on the vector units.
 */
size_t msa_route_workspace_size(msa_dtype dt, int64_t B, int Tq, int Hq, int Hkv,
                                int64_t N, int64_t n_docs, int top_k);

msa_status msa_route(msa_ctx* ctx, msa_dtype dt,
                     const void* Qr, int64_t B, int Tq, int Hq,
                     const void* Krbar, int64_t N, int Hkv,
                     const int64_t* doc_chunk_off, int64_t n_docs, int top_k,
                     int32_t* out_ids, float* out_scores,
                     float* out_chunk, float* out_doc,
                     void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * msa_route_bwd -- gradients of the document scores of msa_route with respect
 * to Qr and K̄r, given dscore = dLoss/dscore.  ([blog] 训练策略: the router is
 * trained by an auxiliary routing loss, a supervised contrastive loss over
 * relevant and irrelevant document blocks, through the document scores;
 * [rev] 核心能力 › 端到端可训练框架.)
 * score[b,doc] = max over the doc's chunks n and tokens t of
 * (1/Hq) sum_h cos(Qr[b,t,h], K̄r[n,h/G]); the max passes its gradient to its
 * arg max (n*, t*) only, the lowest chunk and then the lowest token among
 * equal scores (scores compared in fp32).  With w = dscore[b,doc]/Hq, c_h the
 * cosine of head h at (n*, t*) and ^ the division by the eps-clamped norm:
 *     dQr[b,t*,h] += w (k^ - c_h q^_h) / |q_h|
 *     dK̄r[n*,g]   += w sum_{h in g} (q^_h - c_h k^) / |k|
 * (a norm at or below eps is a constant: the second term drops and |.| is eps).
 *   Qr, Krbar, doc_chunk_off, B, Tq, Hq, N, Hkv, n_docs  as for msa_route;
 *                  Hkv * head_dim a power of two from 64 to 2048; N * Tq < 2^32.
 *   dscore         device float [B][n_docs]; documents with 0 are skipped.
 *   dQr            device float [B][Tq][Hq][d] (written, every element).
 *   dKrbar         device float [N][Hkv][d]: rows of chunks inside some
 *                  document are written (0 where no gradient arrives); rows
 *                  outside every document are untouched.
 *   out_arg        optional device int32 [B][n_docs][2] (8-byte aligned):
 *                  (n*, t*) per document, (-1, -1) where dscore is 0.
 *   workspace      device, >= msa_route_bwd_workspace_size(...) bytes.
 * Every sum runs in a fixed order (no atomics); the result does not depend on
 * scheduling.
 */
size_t msa_route_bwd_workspace_size(int64_t B, int Tq, int Hq, int Hkv, int64_t N, int64_t n_docs);

msa_status msa_route_bwd(msa_ctx* ctx, msa_dtype dt,
                         const void* Qr, int64_t B, int Tq, int Hq,
                         const void* Krbar, int64_t N, int Hkv,
                         const int64_t* doc_chunk_off, int64_t n_docs,
                         const float* dscore, float* dQr, float* dKrbar, int32_t* out_arg,
                         void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * msa_route_time_next -- profiling aid, synchronous.  The next msa_route call
 * on this context has its main chunk-score kernel (the streaming scan, the
 * generic scan, or the matrix-core contraction; not the packing or top-k
 * kernels around it) record `start` when it begins and `stop` when it ends,
 * as part of that kernel's own dispatch, then forgets both; so
 * hipEventElapsedTime(start, stop) is that kernel's duration and timing adds
 * no gap between kernels.  With an empty bank (N = 0) both are recorded back
 * to back.  Both must be events created with timing enabled on the context's
 * device (or both NULL, which clears).  Not for concurrent use of one context
 * from several threads.
 */
msa_status msa_route_time_next(msa_ctx* ctx, hipEvent_t start, hipEvent_t stop);

/*
 * msa_gather -- stage 2b (online): fetch the selected documents' pooled
 * K̄/V̄ rows from the host store.  ([neo] 推論パイプライン: only the selected
 * K̄/V̄ are loaded, content K̄/V̄ live in host memory and are fetched
 * asynchronously when selected; [blog] Memory Parallel: CPU-offloaded K̄/V̄
 * fetched on demand.)
 * For each query b the selected ids are taken in ascending id order and the
 * rows doc_chunk_off[id] .. doc_chunk_off[id+1]-1 of host_KVbar are copied,
 * back to back, to dst_KVmem starting at row mem_off[b]; mem_off[0] = 0 and
 * mem_off[b+1] = mem_off[b] + (rows of query b).  Adjacent selected
 * documents are merged into one copy.  Copies are asynchronous host->device
 * memcpys on `side`: one hipMemcpyAsync per copy, or one hipMemcpyBatchAsync
 * for all of them when the HIP runtime in the process provides that call
 * (and the environment does not set MSA_GATHER_BATCH=0); mem_off_dev (if not
 * NULL) is filled from mem_off_host by the same submission;
 * `done` (if not NULL) is recorded on `side` after the last copy, so the
 * consumer stream can hipStreamWaitEvent on it.
 *   host_KVbar     host store, pinned (hipHostMalloc), rows of row_bytes
 *                  (= 2*Hkv*d*sizeof(dt) for a [N][2][Hkv][d] bank).
 *   n_rows_host    rows in host_KVbar.
 *   doc_chunk_off  host int64[n_docs+1], non-decreasing from 0, last entry
 *                  <= n_rows_host.
 *   ids_host       host int32[B][top_k], ids in [0, n_docs), no duplicate
 *                  within a query.  Read synchronously.
 *   dst_KVmem      device buffer of cap_rows rows.
 *   mem_off_host   host int64[B+1], written synchronously; it is the
 *                  source of the mem_off_dev copy, so keep it unchanged
 *                  until `done` has completed (pinned memory makes that
 *                  copy asynchronous).
 *   mem_off_dev    device int64[B+1] or NULL.
 * Fails with MSA_ERR_INVALID_ARG (nothing enqueued) if the rows do not fit
 * cap_rows or the host store is not pinned.
 */
msa_status msa_gather(const void* host_KVbar, size_t row_bytes, int64_t n_rows_host,
                      const int64_t* doc_chunk_off, int64_t n_docs,
                      const int32_t* ids_host, int64_t B, int top_k,
                      void* dst_KVmem, int64_t cap_rows,
                      int64_t* mem_off_host, int64_t* mem_off_dev,
                      hipStream_t side, hipEvent_t done);

/*
 * msa_gather_device -- stage 2b without a host round trip.  Same result and
 * layout as msa_gather (each query's ids in ascending order, rows back to
 * back, mem_off prefix sums), but the ids stay on the device and a kernel on
 * `stream` reads the selected rows straight from the pinned host store
 * (page-locked host memory is addressable by the GPU) and writes them to
 * dst_KVmem.  ([neo] 推論パイプライン: only the selected K̄/V̄ are loaded from
 * host memory; [blog] Memory Parallel: CPU-offloaded K̄/V̄ fetched on demand.)
 *   host_KVbar     pinned host store (hipHostMalloc), 16-byte aligned, rows
 *                  of row_bytes (a multiple of 16), n_rows_host rows.
 *   doc_chunk_off  device int64[n_docs+1].
 *   ids            device int32[B][top_k] (e.g. msa_route's out_ids).
 *   mem_off        device int64[B+1] output.
 *   workspace      device, >= msa_gather_device_workspace_size(B, top_k,
 *                  cap_rows): the copy plan and one source-row index per
 *                  destination row.
 * B in [1, 1024].  Device-side data are not validated synchronously: an id
 * outside [0, n_docs), or a document whose rows fall outside the host
 * store, contributes no rows; rows beyond cap_rows are dropped (mem_off is
 * clamped to cap_rows).  Every access stays in bounds.
 */
size_t msa_gather_device_workspace_size(int64_t B, int top_k, int64_t cap_rows);

msa_status msa_gather_device(msa_ctx* ctx, const void* host_KVbar, size_t row_bytes,
                             int64_t n_rows_host, const int64_t* doc_chunk_off, int64_t n_docs,
                             const int32_t* ids, int64_t B, int top_k, void* dst_KVmem,
                             int64_t cap_rows, int64_t* mem_off,
                             void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * msa_sparse_attn -- stage 3: GQA attention over [selected K̄/V̄ ; local K/V].
 * ([neo] アーキテクチャ: the compressed K/V are concatenated with the query's
 * local K/V for autoregressive decoding; global RoPE shifts the query start
 * by k so the order is background -> query -> generation; 推論パイプライン
 * third stage.)
 * Positions: local key j (0 <= j < L) sits at q_offset + j; query token i
 * (0 <= i < Tq, the last Tq tokens of the local context) at
 * q_offset + (L - Tq) + i.  Q and K_local are given unrotated and rotated
 * inside; memory keys K̄ are used as stored (they carry document-local RoPE
 * from encoding).  Every memory row is visible to every query token; local
 * key j is visible to query token i iff j <= (L - Tq) + i.  Query head h
 * reads KV head h / (Hq/Hkv).
 *     O[b,i,h] = softmax_j(scale * q~.k~_j) . v_j      (fp32 inside)
 *   Q              device [B][Tq][Hq][d] of dt.
 *   KVmem          device [mem_rows_cap][2][Hkv][d] of dt (msa_gather's
 *                  dst: K̄ then V̄ per row).
 *   mem_off        device int64[B+1]: query b uses rows
 *                  mem_off[b] .. mem_off[b+1]-1 (clamped to
 *                  [0, mem_rows_cap] and to max_rows_per_query rows).
 *   max_rows_per_query  host upper bound of any query's memory rows (sizes
 *                  the launch); 0 is allowed (no memory rows).
 *   K_local, V_local    device [B][L][Hkv][d] of dt; Tq <= L.
 *   q_offset       the global RoPE shift k (normally top_k).
 *   scale          logit scale (normally 1/sqrt(d)).
 *   O              device [B][Tq][Hq][d] of dt.
 *   workspace      device, >= msa_sparse_attn_workspace_size(...) bytes.
 * q_offset + L - 1 must be < max_pos.
 */
size_t msa_sparse_attn_workspace_size(msa_dtype dt, int64_t B, int Tq, int Hq, int Hkv,
                                      int64_t max_rows_per_query, int L);

msa_status msa_sparse_attn(msa_ctx* ctx, msa_dtype dt,
                           const void* Q, int64_t B, int Tq, int Hq,
                           const void* KVmem, const int64_t* mem_off,
                           int64_t mem_rows_cap, int64_t max_rows_per_query,
                           const void* K_local, const void* V_local, int L, int Hkv,
                           int q_offset, float scale, void* O,
                           void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * msa_sparse_attn_noalloc -- msa_sparse_attn without a workspace argument and
 * without any allocation, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments (minus workspace), same kernels, same result
 * bits as msa_sparse_attn.  The split partials and packed key tiles live in
 * a library-held scratch array of MSA_NOALLOC_SCRATCH_BYTES per device, held
 * until the process ends; its device address is taken when the first
 * context on the device is created.  A call whose msa_sparse_attn_workspace_size
 * exceeds that returns MSA_ERR_WORKSPACE (nothing enqueued): decode and
 * short-prompt attention fit, a long prefill does not.  Every call on a
 * device shares that device's array and no part of it needs to start at
 * zero (each kernel writes what it reads); calls that can overlap on one
 * device (other streams, other threads) race on it and must be ordered by
 * the caller.  The call calls no hipMalloc, hipFree or allocating routine.
 */
#define MSA_NOALLOC_SCRATCH_BYTES (16u << 20)

msa_status msa_sparse_attn_noalloc(msa_ctx* ctx, msa_dtype dt,
                                   const void* Q, int64_t B, int Tq, int Hq,
                                   const void* KVmem, const int64_t* mem_off,
                                   int64_t mem_rows_cap, int64_t max_rows_per_query,
                                   const void* K_local, const void* V_local, int L, int Hkv,
                                   int q_offset, float scale, void* O, hipStream_t stream);

/*
 * msa_sparse_attn_lse -- msa_sparse_attn that also saves, per output row, the
 * statistic its backward recomputes the softmax from.  Same arguments, plus
 *   lse            device float [B][Tq][Hq]: natural-log log-sum-exp over the
 *                  row's visible keys of scale * q~.k~ (4-byte aligned).
 * (Training forward; sources as msa_sparse_attn_bwd.)
 */
msa_status msa_sparse_attn_lse(msa_ctx* ctx, msa_dtype dt,
                               const void* Q, int64_t B, int Tq, int Hq,
                               const void* KVmem, const int64_t* mem_off,
                               int64_t mem_rows_cap, int64_t max_rows_per_query,
                               const void* K_local, const void* V_local, int L, int Hkv,
                               int q_offset, float scale, void* O, float* lse,
                               void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * msa_sparse_attn_bwd -- gradients of msa_sparse_attn with respect to Q, the
 * memory rows K̄/V̄ and the local K/V, given dO = dLoss/dO.
 * ([blog] 训练策略: the model is trained with the generation loss, which
 * reaches these inputs through the sparse attention, plus an auxiliary routing
 * loss; [rev] 核心能力 › 端到端可训练框架: retrieval and generation form one
 * differentiable loop.)
 * With P the softmax of a row, dP_j = dO.v_j, D = dO.O, dS_j = P_j (dP_j - D):
 *     dV_j = sum_i P_ij dO_i       dk~_j = scale sum_i dS_ij q~_i
 *     dq~_i = scale sum_j dS_ij k~_j
 * summed over the G query heads of a KV head; dQ and dK_local are the rotated
 * gradients turned back by their RoPE angle; memory keys get dk~ itself.
 *   dt             MSA_BF16 only, head dim 128 (else MSA_ERR_UNSUPPORTED).
 *   Q .. scale     exactly as passed to the forward.
 *   O              device [B][Tq][Hq][d]: the forward's output.
 *   dO             device [B][Tq][Hq][d].
 *   lse            device float [B][Tq][Hq] from msa_sparse_attn_lse.
 *   dQ             device [B][Tq][Hq][d] (written).
 *   dKVmem         device [mem_rows_cap][2][Hkv][d] (dK̄ then dV̄ per row):
 *                  the rows each query uses are written, others untouched;
 *                  the row ranges of different queries must not overlap.
 *   dK_local, dV_local  device [B][L][Hkv][d] (written).
 *   workspace      device, >= msa_sparse_attn_bwd_workspace_size(...) bytes.
 * Gradients are bf16, accumulated in fp32; no atomics, so results do not
 * depend on scheduling.  Outputs must not alias inputs.
 */
size_t msa_sparse_attn_bwd_workspace_size(msa_dtype dt, int64_t B, int Tq, int Hq, int Hkv,
                                          int64_t max_rows_per_query, int L);

msa_status msa_sparse_attn_bwd(msa_ctx* ctx, msa_dtype dt,
                               const void* Q, int64_t B, int Tq, int Hq,
                               const void* KVmem, const int64_t* mem_off,
                               int64_t mem_rows_cap, int64_t max_rows_per_query,
                               const void* K_local, const void* V_local, int L, int Hkv,
                               int q_offset, float scale,
                               const void* O, const void* dO, const float* lse,
                               void* dQ, void* dKVmem, void* dK_local, void* dV_local,
                               void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * msa_gather_attn -- stages 2b and 3 in one call: msa_gather_device of the
 * selected documents' K̄/V̄ rows into dst_KVmem, then msa_sparse_attn over
 * [those rows ; local K/V].  ([neo] 推論パイプライン, Fig. 3: the selected
 * K̄/V̄ are loaded from host memory and concatenated with the local context
 * for the attention; [blog] Memory Parallel: K̄/V̄ live in CPU memory and are
 * fetched when selected.)
 * The local keys need none of the gathered rows, so for decode rows (bf16,
 * d 128, Hq/Hkv in {1, 2, 4, 8}, Tq < 64) their attention runs in the same
 * launch as the PCIe copy, and the memory rows' attention and the merge of
 * both follow it (for one query of one token with Hkv <= 8, the workgroups
 * that copy the memory rows also attend over them, in fp32, so only the
 * merge follows); other shapes run the gather and then the attention.
 * Arguments: those of msa_gather_device (host_KVbar .. mem_off, with
 * B = the queries) followed by those of msa_sparse_attn (Q .. O; KVmem is
 * dst_KVmem and mem_rows_cap is cap_rows), with the same meaning, layout,
 * validation and results: dst_KVmem and mem_off exactly as msa_gather_device
 * writes them, O as msa_sparse_attn computes it (the partial softmaxes are
 * merged in another order, so the bits can differ within rounding).
 * row_bytes must be 2 * Hkv * d * sizeof(dt) (a K̄ row and a V̄ row).
 *   workspace      device, >= msa_gather_attn_workspace_size(...) bytes,
 *                  256-byte aligned; nothing in it needs to start at zero.
 */
size_t msa_gather_attn_workspace_size(msa_dtype dt, int64_t B, int Tq, int Hq, int Hkv, int top_k,
                                      int64_t cap_rows, int64_t max_rows_per_query, int L);

msa_status msa_gather_attn(msa_ctx* ctx, msa_dtype dt,
                           const void* host_KVbar, size_t row_bytes, int64_t n_rows_host,
                           const int64_t* doc_chunk_off, int64_t n_docs,
                           const int32_t* ids, int top_k,
                           void* dst_KVmem, int64_t cap_rows, int64_t* mem_off,
                           const void* Q, int64_t B, int Tq, int Hq, int64_t max_rows_per_query,
                           const void* K_local, const void* V_local, int L, int Hkv,
                           int q_offset, float scale, void* O,
                           void* workspace, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
