"""Stage 3: sparse attention over [selected K̄/V̄ ; local K/V] (test infrastructure).

Sources:
* neo-ai.one MSA article, 全体設計 › アーキテクチャ (Fig. 2): the compressed
  K/V of the selected documents are concatenated with the query's local K/V
  and used for autoregressive decoding; global RoPE shifts the query's start
  index by k, the number of retrieved top-k blocks, so the causal order is
  background -> query -> generation.
* same article, 推論パイプライン (Fig. 3), third stage: sparse generation over
  the assembled context.
* ruixiangma.github.io blog, 三阶段推理流程: generation over the assembled
  sparse context.

Readings taken where the pages are silent:
* k is the integer top_k.  Local key j (0 <= j < L) sits at global position
  k + j; query token i (0 <= i < Tq, the last Tq tokens of the local context)
  sits at k + (L - Tq) + i.  Q and local K are given unrotated and rotated
  here with the rotate-half RoPE.  Memory keys K̄ are used as stored: they
  already carry their document-local RoPE from encoding.
* Mask: every memory row is visible to every query token; local key j is
  visible to query token i iff j <= (L - Tq) + i.  No window, no sink.
* logits scaled by `scale` (1/sqrt(d) in all workloads); softmax with the row
  maximum subtracted; GQA maps query head h to KV head h // (Hq / Hkv).

Parity status: pinned (tests/test_oracle_attention.py): explicit loop form
with complex rotation; with no memory rows it equals torch's CPU
scaled_dot_product_attention on RoPE'd inputs and does not depend on k;
chunk length 1 with every document selected equals full attention over all
document tokens at document-local positions; constant V gives that constant;
Q = 0 gives the mean of the visible V; shifting k by delta equals rotating
the memory keys by -delta.
"""

import cmath
import math

import numpy as np

from .rope import rope


def _attn_one(Q, mem_K, mem_V, K_loc, V_loc, k_off, scale, theta):
    Q = np.asarray(Q, dtype=np.float64)
    Tq, Hq, d = Q.shape
    L, Hkv, _ = np.asarray(K_loc).shape
    M = np.asarray(mem_K).shape[0]
    if Tq > L:
        raise ValueError("query tokens must be the last Tq of the local context")
    G = Hq // Hkv
    q_pos = k_off + (L - Tq) + np.arange(Tq)
    k_pos = k_off + np.arange(L)
    qr = rope(Q, q_pos[:, None], theta)                       # [Tq, Hq, d]
    kr = rope(np.asarray(K_loc, dtype=np.float64), k_pos[:, None], theta)
    mK = np.asarray(mem_K, dtype=np.float64).reshape(M, Hkv, d)
    mV = np.asarray(mem_V, dtype=np.float64).reshape(M, Hkv, d)
    lV = np.asarray(V_loc, dtype=np.float64)
    visible = np.arange(L)[None, :] <= (L - Tq) + np.arange(Tq)[:, None]  # [Tq, L]
    O = np.empty((Tq, Hq, d))
    for h in range(Hq):
        g = h // G
        lm = (qr[:, h, :] @ mK[:, g, :].T) * scale            # [Tq, M]
        ll = (qr[:, h, :] @ kr[:, g, :].T) * scale            # [Tq, L]
        ll = np.where(visible, ll, -np.inf)
        logits = np.concatenate([lm, ll], axis=1)
        mx = np.max(logits, axis=1, keepdims=True)
        p = np.exp(logits - mx)
        p /= np.sum(p, axis=1, keepdims=True)
        vals = np.concatenate([mV[:, g, :], lV[:, g, :]], axis=0)
        O[:, h, :] = p @ vals
    return O


def sparse_attn(Q, mem_K, mem_V, mem_off, K_loc, V_loc, k_off, scale, theta):
    """Batched form.  Q [B, Tq, Hq, d]; mem_K/mem_V [sum M_b, Hkv, d] with the
    rows of query b at mem_off[b]:mem_off[b+1]; K_loc/V_loc [B, L, Hkv, d].
    Returns O [B, Tq, Hq, d] in float64."""
    Q = np.asarray(Q, dtype=np.float64)
    out = np.empty(Q.shape)
    for b in range(Q.shape[0]):
        a, e = int(mem_off[b]), int(mem_off[b + 1])
        out[b] = _attn_one(Q[b], mem_K[a:e], mem_V[a:e], K_loc[b], V_loc[b],
                           k_off, scale, theta)
    return out


def sparse_attn_loops(Q, mem_K, mem_V, K_loc, V_loc, k_off, scale, theta):
    """Explicit-loop form for one query, tiny inputs only.  Rotation by
    complex multiplication, so it shares no RoPE code with rope()."""
    Q = np.asarray(Q, dtype=np.float64)
    Tq, Hq, d = Q.shape
    L, Hkv, _ = np.asarray(K_loc).shape
    M = len(mem_K)
    G = Hq // Hkv
    half = d // 2

    def rot(x, p):
        y = [0.0] * d
        for i in range(half):
            z = complex(x[i], x[i + half]) * cmath.exp(1j * p * math.pow(theta, -2.0 * i / d))
            y[i], y[i + half] = z.real, z.imag
        return y

    O = np.zeros((Tq, Hq, d))
    for i in range(Tq):
        for h in range(Hq):
            g = h // G
            q = rot(Q[i, h], k_off + (L - Tq) + i)
            keys, vals = [], []
            for m in range(M):
                keys.append([float(v) for v in mem_K[m][g]])
                vals.append([float(v) for v in mem_V[m][g]])
            for j in range(L):
                if j <= (L - Tq) + i:
                    keys.append(rot(K_loc[j, g], k_off + j))
                    vals.append([float(v) for v in V_loc[j, g]])
            logits = [scale * sum(q[c] * kk[c] for c in range(d)) for kk in keys]
            mx = max(logits)
            w = [math.exp(x - mx) for x in logits]
            z = sum(w)
            for c in range(d):
                O[i, h, c] = sum(w[n] * vals[n][c] for n in range(len(w))) / z
    return O
