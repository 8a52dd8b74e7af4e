"""Backward of stage 3 (sparse attention) and of the stage 2a document score
(test infrastructure).

Sources:
* ruixiangma.github.io blog, 训练策略: continued pre-training minimises the
  generation loss plus an auxiliary routing loss, a supervised contrastive
  loss that separates relevant from irrelevant document blocks.  The
  generation loss reaches the attention inputs (query, selected K̄/V̄, local
  K/V); the routing loss reaches the routing query Qr and the routing keys K̄r
  through the document scores.
* github-eval-reports review of MSA, 核心能力 › 端到端可训练框架: retrieval and
  generation form one differentiable loop (top-k selection fused with the
  sparse attention, trained jointly).
* neo-ai.one MSA article, 全体設計 › アーキテクチャ (Fig. 2): the forward
  computations being differentiated (cosine routing with head mean and token
  max; attention over [selected K̄/V̄ ; local K/V] with global RoPE).

Readings taken where the pages are silent:
* The pages do not write the contrastive loss out; the backward here starts
  from a given gradient of the loss with respect to the document scores
  (dscore [B, n_docs]) and, for the attention, from dO.
* Attention: the usual softmax backward.  With P the attention weights of a
  query row, dP_j = dO . v_j, D = sum_j P_j dP_j (= dO . O) and
  dS_j = P_j (dP_j - D); the rotated query and key get scale * dS . k~ and
  scale * dS^T . q~, the values P^T . dO.  The rotation is orthogonal, so the
  gradient of an unrotated input is its rotated gradient turned back by the
  same angle (rotation by -angle).  Memory keys are used as stored, so their
  gradient is the rotated-space gradient itself.  GQA: a KV head collects the
  gradients of all query heads that read it.
* Document score D[b, doc] = max over the document's chunks n and the query
  tokens t of (1/Hq) sum_h cos(Qr[b,t,h], K̄r[n, h // G]).  A max passes its
  gradient to the arg max only; among equal values the lowest chunk index,
  then the lowest token, is taken (the same lowest-index rule as the top-k
  tie break).  Off ties the score is differentiable and this is its gradient.
* cos(q, k) = q.k / (max(|q|, eps) * max(|k|, eps)): below eps a norm is a
  constant and contributes no derivative.
* The saved forward statistic of a query row is the natural-log
  log-sum-exp of its visible scaled logits.
* Pooling (neo-ai.one article, アーキテクチャ: chunk means of the documents'
  K/V/Kr, keys rotated at document-local positions): a chunk mean passes
  1/count of its gradient to each of its rows; a key row's share is turned
  back by its document-local angle.

Parity status: pinned (tests/test_oracle_backward.py): every element of every
gradient against central finite differences of the pinned forward oracles on
tiny inputs; the key-translation identity (each softmax row's dS sums to 0,
so the rotated key gradients of a query row sum to 0); the value-gradient sum
(rows of P sum to 1); the bilinear identity <Q, dQ> = <K, dK> over all keys;
the scale invariance of the cosine (<q, dq> = 0, <k, dk> = 0); log-sum-exp
closed forms (Q = 0 gives log of the visible count; it reproduces the forward
output); the pooling backward against finite differences of encode_pool and
by its chunk sums (the rows of a chunk sum back to the pooled gradient).
"""

import numpy as np

from .attention import sparse_attn
from .encode import chunk_offsets
from .rope import rope
from .route import EPS


def _rows(Q, mem_K, mem_V, K_loc, V_loc, k_off, scale, theta):
    """Rotated queries, the key/value rows of each KV head ([memory ; local])
    and the visibility mask of one query, all float64."""
    Q = np.asarray(Q, dtype=np.float64)
    Tq, Hq, d = Q.shape
    L, Hkv, _ = np.asarray(K_loc).shape
    M = np.asarray(mem_K).shape[0]
    q_pos = k_off + (L - Tq) + np.arange(Tq)
    k_pos = k_off + np.arange(L)
    qr = rope(Q, q_pos[:, None], theta)
    kr = rope(np.asarray(K_loc, dtype=np.float64), k_pos[:, None], theta)
    mK = np.asarray(mem_K, dtype=np.float64).reshape(M, Hkv, d)
    mV = np.asarray(mem_V, dtype=np.float64).reshape(M, Hkv, d)
    lV = np.asarray(V_loc, dtype=np.float64)
    keys = np.concatenate([mK, kr], axis=0)                  # [M + L, Hkv, d]
    vals = np.concatenate([mV, lV], axis=0)
    vis_loc = np.arange(L)[None, :] <= (L - Tq) + np.arange(Tq)[:, None]
    visible = np.concatenate([np.ones((Tq, M), dtype=bool), vis_loc], axis=1)
    return qr, keys, vals, visible, q_pos, k_pos, M


def _softmax_rows(logits, visible):
    z = np.where(visible, logits, -np.inf)
    mx = np.max(z, axis=1, keepdims=True)
    p = np.exp(z - mx)
    return p / np.sum(p, axis=1, keepdims=True), mx[:, 0] + np.log(np.sum(np.exp(z - mx), axis=1))


def sparse_attn_lse(Q, mem_K, mem_V, mem_off, K_loc, V_loc, k_off, scale, theta):
    """lse[b, i, h] = log sum over visible keys j of exp(scale * q~_i . k~_j)."""
    Q = np.asarray(Q, dtype=np.float64)
    B, Tq, Hq, d = Q.shape
    Hkv = np.asarray(K_loc).shape[2]
    G = Hq // Hkv
    out = np.empty((B, Tq, Hq))
    for b in range(B):
        a, e = int(mem_off[b]), int(mem_off[b + 1])
        qr, keys, _, visible, _, _, _ = _rows(Q[b], mem_K[a:e], mem_V[a:e], K_loc[b], V_loc[b],
                                              k_off, scale, theta)
        for h in range(Hq):
            _, lse = _softmax_rows(scale * (qr[:, h, :] @ keys[:, h // G, :].T), visible)
            out[b, :, h] = lse
    return out


def sparse_attn_bwd(Q, mem_K, mem_V, mem_off, K_loc, V_loc, k_off, scale, theta, dO):
    """Gradients of sum(dO * O) for O = sparse_attn(...).

    Shapes as sparse_attn; dO [B, Tq, Hq, d].  Returns float64
    (dQ [B, Tq, Hq, d], dmem_K and dmem_V shaped like mem_K (rows no query
    uses stay 0), dK_loc [B, L, Hkv, d], dV_loc [B, L, Hkv, d])."""
    Q = np.asarray(Q, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    B, Tq, Hq, d = Q.shape
    L, Hkv = np.asarray(K_loc).shape[1:3]
    G = Hq // Hkv
    n_mem = np.asarray(mem_K).shape[0]
    dQ = np.zeros(Q.shape)
    dmK = np.zeros((n_mem, Hkv, d))
    dmV = np.zeros((n_mem, Hkv, d))
    dKl = np.zeros((B, L, Hkv, d))
    dVl = np.zeros((B, L, Hkv, d))
    for b in range(B):
        a, e = int(mem_off[b]), int(mem_off[b + 1])
        qr, keys, vals, visible, q_pos, k_pos, M = _rows(Q[b], mem_K[a:e], mem_V[a:e], K_loc[b],
                                                         V_loc[b], k_off, scale, theta)
        dqr = np.zeros(qr.shape)
        dkeys = np.zeros(keys.shape)
        dvals = np.zeros(vals.shape)
        for h in range(Hq):
            g = h // G
            P, _ = _softmax_rows(scale * (qr[:, h, :] @ keys[:, g, :].T), visible)   # [Tq, M + L]
            dPm = dO[b, :, h, :] @ vals[:, g, :].T                                   # dP_ij = dO_i . v_j
            Drow = np.sum(P * dPm, axis=1, keepdims=True)
            dS = P * (dPm - Drow)
            dqr[:, h, :] = scale * (dS @ keys[:, g, :])
            dkeys[:, g, :] += scale * (dS.T @ qr[:, h, :])
            dvals[:, g, :] += P.T @ dO[b, :, h, :]
        dQ[b] = rope(dqr, -q_pos[:, None], theta)          # rotation back by -angle
        dmK[a:e] += dkeys[:M]
        dmV[a:e] += dvals[:M]
        dKl[b] = rope(dkeys[M:], -k_pos[:, None], theta)
        dVl[b] = dvals[M:]
    return dQ, dmK, dmV, dKl, dVl


def sparse_attn_bwd_sampled(Q, mem_K, mem_V, K_loc, V_loc, k_off, scale, theta, dO, g, q_rows, key_rows,
                            row_block=1024):
    """Selected outputs of sparse_attn_bwd for one query (no batch axis) and
    one KV head g, for sizes where the full gradients are too large to form:
    dQ[q_rows, h] for the G query heads h of g, and dK, dV of the keys
    key_rows (indices into [memory ; local]; memory rows as stored, local
    keys turned back by their angle).  Every query row's softmax is formed
    whole; rows are visited row_block at a time only to bound memory.
    Returns float64 (dQ [len(q_rows), G, d], dK [len(key_rows), d],
    dV [len(key_rows), d])."""
    Q = np.asarray(Q, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    Tq, Hq, d = Q.shape
    L, Hkv = np.asarray(K_loc).shape[:2]
    G = Hq // Hkv
    qr, keys, vals, visible, q_pos, k_pos, M = _rows(Q, mem_K, mem_V, K_loc, V_loc, k_off, scale, theta)
    kg, vg = keys[:, g, :], vals[:, g, :]
    q_rows = np.asarray(q_rows)
    key_rows = np.asarray(key_rows)
    dq = np.zeros((len(q_rows), G, d))
    dk = np.zeros((len(key_rows), d))
    dv = np.zeros((len(key_rows), d))
    for hh in range(G):
        h = g * G + hh
        for r0 in range(0, Tq, row_block):
            r1 = min(Tq, r0 + row_block)
            P, _ = _softmax_rows(scale * (qr[r0:r1, h, :] @ kg.T), visible[r0:r1])
            dPm = dO[r0:r1, h, :] @ vg.T
            dS = P * (dPm - np.sum(P * dPm, axis=1, keepdims=True))
            dk += scale * (dS[:, key_rows].T @ qr[r0:r1, h, :])
            dv += P[:, key_rows].T @ dO[r0:r1, h, :]
            sel = (q_rows >= r0) & (q_rows < r1)
            if np.any(sel):
                dq[sel, hh] = scale * (dS[q_rows[sel] - r0] @ kg)
    dq = rope(dq, -q_pos[q_rows][:, None], theta)
    loc = key_rows >= M
    if np.any(loc):
        dk[loc] = rope(dk[loc], -k_pos[key_rows[loc] - M], theta)
    return dq, dk, dv


def pair_scores(Qr, Krbar, eps=EPS):
    """s[b, n, t] = (1/Hq) sum_h cos(Qr[b,t,h], K̄r[n, h // G]): the score of
    every (chunk, token) pair, head sum in head order."""
    Qr = np.asarray(Qr, dtype=np.float64)
    Kr = np.asarray(Krbar, dtype=np.float64)
    B, T, Hq, d = Qr.shape
    Hkv = Kr.shape[1]
    G = Hq // Hkv
    nq = np.maximum(np.sqrt(np.sum(Qr * Qr, axis=-1, keepdims=True)), eps)
    nk = np.maximum(np.sqrt(np.sum(Kr * Kr, axis=-1, keepdims=True)), eps)
    Qn, Kn = Qr / nq, Kr / nk
    out = np.empty((B, Kr.shape[0], T))
    for b in range(B):
        s = np.zeros((Kr.shape[0], T))
        for h in range(Hq):
            s += Kn[:, h // G, :] @ Qn[b, :, h, :].T
        out[b] = s / Hq
    return out


def doc_score_argmax(Qr, Krbar, doc_chunk_off, eps=EPS):
    """Document scores with the (chunk, token) that attains each.

    Returns score [B, n_docs], arg_chunk [B, n_docs] (global chunk row),
    arg_tok [B, n_docs]; ties go to the lowest chunk, then the lowest token."""
    off = np.asarray(doc_chunk_off, dtype=np.int64)
    S = pair_scores(Qr, Krbar, eps)
    B, _, T = S.shape
    n_docs = len(off) - 1
    score = np.empty((B, n_docs))
    arg_c = np.empty((B, n_docs), dtype=np.int64)
    arg_t = np.empty((B, n_docs), dtype=np.int64)
    for b in range(B):
        s = S[b]
        for doc in range(n_docs):
            blk = s[off[doc]:off[doc + 1]]
            flat = int(np.argmax(blk))                          # first max in (chunk, token) order
            n, t = divmod(flat, T)
            score[b, doc] = blk[n, t]
            arg_c[b, doc] = off[doc] + n
            arg_t[b, doc] = t
    return score, arg_c, arg_t


def _cos_grads(q, k, eps):
    """d cos(q, k) / dq and / dk for the eps-clamped cosine."""
    a, c = np.sqrt(q @ q), np.sqrt(k @ k)
    nq, nk = max(a, eps), max(c, eps)
    dot = q @ k
    dq = k / (nq * nk)
    dk = q / (nq * nk)
    if a > eps:
        dq = dq - dot / (nq ** 3 * nk) * q
    if c > eps:
        dk = dk - dot / (nq * nk ** 3) * k
    return dq, dk


def route_score_bwd(Qr, Krbar, doc_chunk_off, dscore, eps=EPS):
    """Gradients of sum(dscore * score) for score = doc_score_argmax(...)[0].

    Returns float64 (dQr [B, T, Hq, d], dKrbar [N, Hkv, d])."""
    Qr = np.asarray(Qr, dtype=np.float64)
    Kr = np.asarray(Krbar, dtype=np.float64)
    dscore = np.asarray(dscore, dtype=np.float64)
    B, T, Hq, d = Qr.shape
    Hkv = Kr.shape[1]
    G = Hq // Hkv
    _, arg_c, arg_t = doc_score_argmax(Qr, Kr, doc_chunk_off, eps)
    dQr = np.zeros(Qr.shape)
    dKr = np.zeros(Kr.shape)
    for b in range(B):
        for doc in range(dscore.shape[1]):
            w = dscore[b, doc] / Hq
            if w == 0.0:
                continue
            n, t = arg_c[b, doc], arg_t[b, doc]
            for h in range(Hq):
                gq, gk = _cos_grads(Qr[b, t, h], Kr[n, h // G], eps)
                dQr[b, t, h] += w * gq
                dKr[n, h // G] += w * gk
    return dQr, dKr


def sparse_attn_loss(Q, mem_K, mem_V, mem_off, K_loc, V_loc, k_off, scale, theta, dO):
    """sum(dO * O): the scalar whose gradient sparse_attn_bwd returns."""
    O = sparse_attn(Q, mem_K, mem_V, mem_off, K_loc, V_loc, k_off, scale, theta)
    return float(np.sum(np.asarray(dO, dtype=np.float64) * O))


def encode_pool_bwd(dKbar, dVbar, dKrbar, doc_tok_off, chunk_len, theta):
    """Gradients of sum(dKbar * Kbar + dVbar * Vbar + dKrbar * Krbar) for
    (Kbar, Vbar, Krbar) = encode_pool(K, V, Kr, ...): (dK, dV, dKr), each
    float64 [T, Hkv, d]."""
    dKbar = np.asarray(dKbar, dtype=np.float64)
    dVbar = np.asarray(dVbar, dtype=np.float64)
    dKrbar = np.asarray(dKrbar, dtype=np.float64)
    doc_tok_off = np.asarray(doc_tok_off, dtype=np.int64)
    off = chunk_offsets(doc_tok_off, chunk_len)
    T = int(doc_tok_off[-1])
    shape = (T,) + dKbar.shape[1:]
    dK, dV, dKr = np.zeros(shape), np.zeros(shape), np.zeros(shape)
    for doc in range(len(doc_tok_off) - 1):
        s, e = int(doc_tok_off[doc]), int(doc_tok_off[doc + 1])
        j = np.arange(e - s)                          # document-local positions
        row = int(off[doc]) + j // chunk_len          # the chunk row of each token
        cnt = np.minimum((j // chunk_len) * chunk_len + chunk_len, e - s) - (j // chunk_len) * chunk_len
        w = (1.0 / cnt)[:, None, None]
        dK[s:e] = rope(dKbar[row] * w, -j[:, None], theta)
        dV[s:e] = dVbar[row] * w
        dKr[s:e] = dKrbar[row] * w
    return dK, dV, dKr
