"""Stage 1 (offline): document-wise RoPE + chunk mean-pooling (test infrastructure).

Sources:
* neo-ai.one MSA article, 全体設計 › アーキテクチャ (Fig. 2): each document's
  latent state (K, V, Kr) is compressed by chunk-wise mean pooling; positions
  restart at 0 in every document (parallel / document-wise RoPE).
* same article, 推論パイプライン (Fig. 3), first stage: a forward pass over
  the corpus caches the chunk-pooled (K̄, V̄, K̄r).
* ruixiangma.github.io blog, 方法 › 稀疏注意力机制 (split each document into
  fixed-length chunks, mean-pool) and 文档级RoPE (independent start id 0).
* ai-papers.net MSA summary, MSAの提案手法 (fixed-length chunks, mean pooling).

Readings taken where the pages are silent:
* Chunk length c is a parameter.  A document of n tokens has ceil(n / c)
  chunks; the last one is the mean of the rows it actually has.
* RoPE is applied to K before pooling (the cached K of a forward pass is the
  rotated one), at the token's index inside its document (not the chunk
  index).  V and the routing key Kr carry no RoPE.
* Sum in row order, divide by the actual row count.  Chunks of document d
  occupy global chunk rows doc_chunk_off[d] .. doc_chunk_off[d+1]-1, with
  doc_chunk_off the prefix sum of the per-document chunk counts.

Parity status: pinned (tests/test_oracle_encode.py): the loop version with
complex-number rotation agrees; V̄ and K̄r equal np.mean of the chunk rows;
chunk_len 1 gives K̄ = RoPE(K) and the first row of each document equals raw K
bit for bit; moving a document to another offset leaves its pooled rows bit
identical.
"""

import cmath
import math

import numpy as np

from .rope import rope


def chunk_counts(lengths, chunk_len):
    lengths = np.asarray(lengths, dtype=np.int64)
    return (lengths + chunk_len - 1) // chunk_len


def chunk_offsets(doc_tok_off, chunk_len):
    """doc_chunk_off[n_docs+1] = prefix sum of ceil(len_d / c)."""
    doc_tok_off = np.asarray(doc_tok_off, dtype=np.int64)
    counts = chunk_counts(np.diff(doc_tok_off), chunk_len)
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def chunk_mean(X, doc_tok_off, chunk_len):
    """Plain chunk means of X[T, ...] (the V̄ and K̄r part of encode_pool)."""
    X = np.asarray(X, dtype=np.float64)
    doc_tok_off = np.asarray(doc_tok_off, dtype=np.int64)
    lens = np.diff(doc_tok_off)
    if np.any(lens < 1):
        raise ValueError("every document needs at least one token")
    off = chunk_offsets(doc_tok_off, chunk_len)
    out = np.empty((int(off[-1]),) + X.shape[1:])
    for doc in range(len(lens)):
        s, e = int(doc_tok_off[doc]), int(doc_tok_off[doc + 1])
        starts = np.arange(0, e - s, chunk_len)
        cnt = np.minimum(starts + chunk_len, e - s) - starts
        shape = (-1,) + (1,) * (X.ndim - 1)
        out[off[doc]:off[doc + 1]] = np.add.reduceat(X[s:e], starts, axis=0) / cnt.reshape(shape)
    return out


def encode_pool(K, V, Kr, doc_tok_off, chunk_len, theta):
    """K, V, Kr: float64 [T, Hkv, d].  Returns (Kbar, Vbar, Krbar), each
    float64 [N, Hkv, d] with N = sum_d ceil(len_d / chunk_len)."""
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Kr = np.asarray(Kr, dtype=np.float64)
    doc_tok_off = np.asarray(doc_tok_off, dtype=np.int64)
    if chunk_len < 1:
        raise ValueError("chunk_len must be >= 1")
    lens = np.diff(doc_tok_off)
    if np.any(lens < 1):
        raise ValueError("every document needs at least one token")
    off = chunk_offsets(doc_tok_off, chunk_len)
    N = int(off[-1])
    _, H, d = K.shape
    Kb = np.empty((N, H, d))
    Vb = np.empty((N, H, d))
    Rb = np.empty((N, H, d))
    for doc in range(len(lens)):
        s, e = int(doc_tok_off[doc]), int(doc_tok_off[doc + 1])
        pos = np.arange(e - s)                       # document-local positions
        k_rot = rope(K[s:e], pos[:, None], theta)     # [n, H, d]
        starts = np.arange(0, e - s, chunk_len)
        cnt = np.minimum(starts + chunk_len, e - s) - starts
        c0 = int(off[doc])
        c1 = c0 + len(starts)
        Kb[c0:c1] = np.add.reduceat(k_rot, starts, axis=0) / cnt[:, None, None]
        Vb[c0:c1] = np.add.reduceat(V[s:e], starts, axis=0) / cnt[:, None, None]
        Rb[c0:c1] = np.add.reduceat(Kr[s:e], starts, axis=0) / cnt[:, None, None]
    return Kb, Vb, Rb


def encode_pool_loops(K, V, Kr, doc_tok_off, chunk_len, theta):
    """Scalar-loop form for tiny inputs.  Rotation by complex multiplication,
    (x_i + j x_{i+d/2}) * exp(j * pos * theta^(-2i/d)), so it shares no RoPE
    code with rope()."""
    K = np.asarray(K, dtype=np.float64)
    T, H, d = K.shape
    half = d // 2
    out_k, out_v, out_r = [], [], []
    for doc in range(len(doc_tok_off) - 1):
        s, e = int(doc_tok_off[doc]), int(doc_tok_off[doc + 1])
        r0 = s
        while r0 < e:
            r1 = min(r0 + chunk_len, e)
            ck = [[0.0] * d for _ in range(H)]
            cv = [[0.0] * d for _ in range(H)]
            cr = [[0.0] * d for _ in range(H)]
            for r in range(r0, r1):
                p = r - s
                for h in range(H):
                    for i in range(half):
                        z = complex(K[r, h, i], K[r, h, i + half])
                        z *= cmath.exp(1j * (p * math.pow(theta, -2.0 * i / d)))
                        ck[h][i] += z.real
                        ck[h][i + half] += z.imag
                    for i in range(d):
                        cv[h][i] += float(V[r, h, i])
                        cr[h][i] += float(Kr[r, h, i])
            n = r1 - r0
            out_k.append([[x / n for x in row] for row in ck])
            out_v.append([[x / n for x in row] for row in cv])
            out_r.append([[x / n for x in row] for row in cr])
            r0 = r1
    return np.array(out_k), np.array(out_v), np.array(out_r)
