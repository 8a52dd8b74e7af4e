"""Stage 2a (online): cosine routing, document score, top-k (test infrastructure).

Sources:
* neo-ai.one MSA article, 全体設計 › アーキテクチャ (Fig. 2): the routing
  projector scores relevance by cosine similarity, averaged over attention
  heads and then maximised over tokens, and selects the top-k documents.
* same article, 推論パイプライン (Fig. 3), second stage: the query is projected
  to Qr, matched against K̄r, and the top-k is selected.
* ruixiangma.github.io blog, 方法 › 稀疏注意力机制: top-k most relevant
  documents by cosine similarity between the query and the memory.
* github-eval-reports review of MSA, 核心模块: head mean first, then token max.

Readings taken where the pages are silent:
* cos(q, k) = q.k / (max(|q|, eps) * max(|k|, eps)), eps = 1e-8, so a zero
  vector scores 0 instead of dividing by zero.
* GQA: query head h is compared with routing-key head h // (Hq / Hkv); the
  mean runs over all Hq query heads, summed in head order.  It is the mean of
  the per-head cosines, not the cosine of a head-averaged vector.
* "max over tokens" is the max over the query tokens t; the document score is
  then the max over the document's chunks.
* The routing key consumed is the stored K̄r (already rounded to the storage
  dtype), widened to float64.
* Top-k: documents sorted by (score descending, doc id ascending), first k
  kept, so ties go to the lowest doc id.  Inputs are finite.

Parity status: pinned (tests/test_oracle_route.py): brute-force scalar loops,
invariance of scores under scaling by powers of two (bit exact), permutation
equivariance, tie to the lowest id, exhaustive top-k against a textbook full
sort, and recovery of planted documents.
"""

import math

import numpy as np

EPS = 1e-8


def _unit(x, eps=EPS):
    n = np.maximum(np.sqrt(np.sum(x * x, axis=-1, keepdims=True)), eps)
    return x / n


def chunk_scores(Qr, Krbar, eps=EPS):
    """Qr float64 [B, T, Hq, d]; Krbar float64 [N, Hkv, d] (any subset of the
    bank's rows).  Returns c[B, N] = max_t (1/Hq) sum_h cos(Qr[b,t,h],
    Krbar[n, h // G]).  The matmul per head is a library dot product; the
    head sum runs in head order."""
    Qr = np.asarray(Qr, dtype=np.float64)
    Krbar = np.asarray(Krbar, dtype=np.float64)
    B, T, Hq, d = Qr.shape
    N, Hkv, d2 = Krbar.shape
    if d != d2 or Hq % Hkv:
        raise ValueError("shape mismatch")
    G = Hq // Hkv
    Qn = _unit(Qr, eps)
    Kn = _unit(Krbar, eps)
    out = np.empty((B, N))
    for b in range(B):
        s = np.zeros((T, N))
        for h in range(Hq):
            s += Qn[b, :, h, :] @ Kn[:, h // G, :].T
        out[b] = np.max(s / Hq, axis=0)
    return out


def chunk_scores_loops(Qr, Krbar, eps=EPS):
    """Scalar triple loop over (t, h, n) for tiny inputs."""
    Qr = np.asarray(Qr, dtype=np.float64)
    Krbar = np.asarray(Krbar, dtype=np.float64)
    B, T, Hq, d = Qr.shape
    N, Hkv, _ = Krbar.shape
    G = Hq // Hkv
    out = np.full((B, N), -math.inf)
    for b in range(B):
        for n in range(N):
            for t in range(T):
                acc = 0.0
                for h in range(Hq):
                    q = Qr[b, t, h]
                    k = Krbar[n, h // G]
                    dot = sum(float(q[i]) * float(k[i]) for i in range(d))
                    nq = math.sqrt(sum(float(v) * float(v) for v in q))
                    nk = math.sqrt(sum(float(v) * float(v) for v in k))
                    acc += dot / (max(nq, eps) * max(nk, eps))
                out[b, n] = max(out[b, n], acc / Hq)
    return out


def doc_scores(c, doc_chunk_off):
    """D[b, doc] = max of c[b, n] over the document's chunk rows."""
    c = np.asarray(c, dtype=np.float64)
    off = np.asarray(doc_chunk_off, dtype=np.int64)
    if np.any(np.diff(off) < 1):
        raise ValueError("every document needs at least one chunk")
    return np.maximum.reduceat(c, off[:-1], axis=-1)


def topk_docs(D, k):
    """Ids [B, k] and scores [B, k]: sort by (-D, id), keep the first k."""
    D = np.asarray(D, dtype=np.float64)
    B, n_docs = D.shape
    if not 1 <= k <= n_docs:
        raise ValueError("need 1 <= k <= n_docs")
    ids = np.empty((B, k), dtype=np.int64)
    for b in range(B):
        order = np.lexsort((np.arange(n_docs), -D[b]))
        ids[b] = order[:k]
    return ids, np.take_along_axis(D, ids, axis=1)


def route(Qr, Krbar, doc_chunk_off, k, eps=EPS):
    """Full routing: returns (ids, top scores, chunk scores c, doc scores D)."""
    c = chunk_scores(Qr, Krbar, eps)
    D = doc_scores(c, doc_chunk_off)
    ids, sc = topk_docs(D, k)
    return ids, sc, c, D
