"""Pins of the oracle's backward: attention (dQ, dK̄, dV̄, dK_local,
dV_local), its saved log-sum-exp, and the document-score gradient (dQr, dK̄r).

The gradients are pinned element by element against central finite
differences of the forward oracles, which have their own pins, and by
identities that a dropped term, a wrong sign, a wrong rotation direction or a
transposed operand breaks."""

import math

import numpy as np
import pytest

import oracle
from oracle import backward as bw

THETA = 1e4


def _attn_case(rng, B=2, Tq=3, L=5, Hq=4, Hkv=2, d=8, M=(3, 2)):
    mem_off = np.concatenate([[0], np.cumsum(M)]).astype(np.int64)
    n = int(mem_off[-1])
    return dict(Q=rng.standard_normal((B, Tq, Hq, d)), mem_K=rng.standard_normal((n, Hkv, d)),
                mem_V=rng.standard_normal((n, Hkv, d)), mem_off=mem_off,
                K_loc=rng.standard_normal((B, L, Hkv, d)), V_loc=rng.standard_normal((B, L, Hkv, d)),
                k_off=4, scale=1.0 / math.sqrt(d), theta=THETA)


NAMES = ["Q", "mem_K", "mem_V", "K_loc", "V_loc"]


def _fd(loss, arr, h=1e-5):
    g = np.zeros(arr.shape)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = arr[i]
        arr[i] = old + h
        up = loss()
        arr[i] = old - h
        dn = loss()
        arr[i] = old
        g[i] = (up - dn) / (2 * h)
    return g


@pytest.mark.parametrize("shape", [
    dict(),                                   # GQA 2, memory rows for both queries
    dict(Hq=2, Hkv=2, M=(0, 4)),              # no GQA, one query without memory
    dict(Tq=4, L=4, Hq=4, Hkv=1, M=(2, 1)),   # every local key causal, GQA 4
])
def test_attention_gradients_match_finite_differences(shape):
    rng = np.random.default_rng(len(str(shape)))
    c = _attn_case(rng, **shape)
    dO = rng.standard_normal(c["Q"].shape)
    grads = bw.sparse_attn_bwd(**c, dO=dO)
    for name, got in zip(NAMES, grads):
        fd = _fd(lambda: bw.sparse_attn_loss(**c, dO=dO), c[name])
        np.testing.assert_allclose(got, fd, rtol=1e-6, atol=1e-8, err_msg=name)


def test_attention_gradient_identities():
    rng = np.random.default_rng(7)
    B, Tq, L, Hq, Hkv, d = 2, 5, 9, 8, 2, 16
    c = _attn_case(rng, B, Tq, L, Hq, Hkv, d, M=(6, 3))
    dO = rng.standard_normal(c["Q"].shape)
    dQ, dmK, dmV, dKl, dVl = bw.sparse_attn_bwd(**c, dO=dO)
    G = Hq // Hkv
    off = c["mem_off"]
    for b in range(B):
        k_pos = c["k_off"] + np.arange(L)
        dk_rot = oracle.rope(dKl[b], k_pos[:, None], THETA)      # back to the rotated key space
        tot_k = dmK[off[b]:off[b + 1]].sum(axis=0) + dk_rot.sum(axis=0)
        np.testing.assert_allclose(tot_k, 0.0, atol=1e-10)     # each dS row sums to 0
        tot_v = dmV[off[b]:off[b + 1]].sum(axis=0) + dVl[b].sum(axis=0)
        want_v = dO[b].reshape(Tq, Hkv, G, d).sum(axis=(0, 2))  # rows of P sum to 1
        np.testing.assert_allclose(tot_v, want_v, rtol=1e-10, atol=1e-10)
    # logits are bilinear in (q, k): scaling Q or every key by a changes the loss alike
    lhs = np.sum(c["Q"] * dQ)
    rhs = np.sum(c["mem_K"] * dmK) + np.sum(c["K_loc"] * dKl)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-10)


def test_sampled_attention_gradients_match_the_full_ones():
    rng = np.random.default_rng(13)
    B, Tq, L, Hq, Hkv, d, M = 1, 11, 14, 8, 2, 16, 5
    c = _attn_case(rng, B, Tq, L, Hq, Hkv, d, M=(M,))
    dO = rng.standard_normal(c["Q"].shape)
    dQ, dmK, dmV, dKl, dVl = bw.sparse_attn_bwd(**c, dO=dO)
    q_rows = np.array([0, 3, 4, 10])
    key_rows = np.array([0, 4, 5, 9, 18])                  # memory rows and local keys
    for g in range(Hkv):
        dq, dk, dv = bw.sparse_attn_bwd_sampled(c["Q"][0], c["mem_K"], c["mem_V"], c["K_loc"][0], c["V_loc"][0],
                                                c["k_off"], c["scale"], THETA, dO[0], g, q_rows, key_rows,
                                                row_block=4)
        G = Hq // Hkv
        np.testing.assert_allclose(dq, dQ[0][q_rows][:, g * G:(g + 1) * G], rtol=1e-11, atol=1e-13)
        allk = np.concatenate([dmK[:, g], dKl[0, :, g]])
        allv = np.concatenate([dmV[:, g], dVl[0, :, g]])
        np.testing.assert_allclose(dk, allk[key_rows], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(dv, allv[key_rows], rtol=1e-11, atol=1e-13)


def test_attention_single_key_row_has_no_query_gradient():
    # Tq = L and no memory: query 0 sees only local key 0, a softmax over one
    # key is constantly 1, so dQ of token 0 is 0 and dV of key 0 collects dO.
    rng = np.random.default_rng(3)
    c = _attn_case(rng, B=1, Tq=4, L=4, Hq=2, Hkv=2, d=8, M=(0,))
    dO = rng.standard_normal(c["Q"].shape)
    dQ, _, _, _, dVl = bw.sparse_attn_bwd(**c, dO=dO)
    np.testing.assert_allclose(dQ[0, 0], 0.0, atol=1e-14)
    assert np.abs(dQ[0, 1:]).max() > 1e-3


def test_lse_closed_forms():
    rng = np.random.default_rng(11)
    c = _attn_case(rng, B=2, Tq=3, L=5, M=(3, 2))
    c["Q"][:] = 0.0
    lse = bw.sparse_attn_lse(**c)
    for b, M in enumerate((3, 2)):
        for i in range(3):
            np.testing.assert_allclose(lse[b, i], math.log(M + (5 - 3) + i + 1), rtol=1e-14)
    # one visible key at the same position as the query: rotation cancels
    c = _attn_case(rng, B=1, Tq=4, L=4, Hq=2, Hkv=2, d=8, M=(0,))
    lse = bw.sparse_attn_lse(**c)
    want = c["scale"] * np.sum(c["Q"][0, 0] * c["K_loc"][0, 0], axis=-1)
    np.testing.assert_allclose(lse[0, 0], want, rtol=1e-12)
    # bounds: max logit <= lse <= max logit + log(count), and lse grows with the scale
    c = _attn_case(rng)
    big = dict(c, scale=40.0)
    lse_b = bw.sparse_attn_lse(**big)
    lse_s = bw.sparse_attn_lse(**c)
    assert np.all(np.isfinite(lse_b)) and np.all(lse_b > lse_s)


def test_lse_reproduces_forward_output():
    # O = sum_j exp(logit_j - lse) v_j: with V = one-hot columns the output is
    # the attention weight itself, so the weights the forward oracle uses must
    # sum to exp(logsumexp - lse) = 1 and match exp(logit - lse) key by key.
    rng = np.random.default_rng(5)
    B, Tq, L, Hq, Hkv, d, M = 1, 2, 3, 2, 1, 8, 4
    c = _attn_case(rng, B, Tq, L, Hq, Hkv, d, M=(M,))
    lse = bw.sparse_attn_lse(**c)
    qrot = oracle.rope(c["Q"][0], (c["k_off"] + L - Tq + np.arange(Tq))[:, None], THETA)
    for j in range(M):                 # memory keys are used as stored
        mV = np.zeros_like(c["mem_V"])
        mV[j, :, 0] = 1.0
        w = oracle.sparse_attn(c["Q"], c["mem_K"], mV, c["mem_off"], c["K_loc"], np.zeros_like(c["V_loc"]),
                               c["k_off"], c["scale"], THETA)[0, :, :, 0]      # [Tq, Hq] weight of key j
        logit = c["scale"] * np.einsum("thd,d->th", qrot, c["mem_K"][j, 0])
        np.testing.assert_allclose(w, np.exp(logit - lse[0]), rtol=1e-10)


def _route_case(rng, B=2, T=3, Hq=4, Hkv=2, d=8, lens=(2, 1, 4)):
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return (rng.standard_normal((B, T, Hq, d)), rng.standard_normal((int(off[-1]), Hkv, d)), off)


def test_doc_score_argmax_matches_forward_scores():
    rng = np.random.default_rng(2)
    Qr, Kr, off = _route_case(rng)
    score, ac, at = bw.doc_score_argmax(Qr, Kr, off)
    np.testing.assert_allclose(score, oracle.doc_scores(oracle.chunk_scores(Qr, Kr), off), rtol=1e-14)
    s = oracle.chunk_scores_loops(Qr[:, :, :, :], Kr)      # [B, N] max over tokens
    for b in range(Qr.shape[0]):
        for doc in range(len(off) - 1):
            assert off[doc] <= ac[b, doc] < off[doc + 1]
            np.testing.assert_allclose(s[b, ac[b, doc]], score[b, doc], rtol=1e-12)
            one = oracle.chunk_scores_loops(Qr[b:b + 1, at[b, doc]:at[b, doc] + 1], Kr[ac[b, doc]:ac[b, doc] + 1])
            np.testing.assert_allclose(one[0, 0], score[b, doc], rtol=1e-12)


def test_pair_scores_reduce_to_the_forward_chunk_scores():
    rng = np.random.default_rng(6)
    Qr, Kr, off = _route_case(rng, B=2, T=4, lens=(3, 2))
    S = bw.pair_scores(Qr, Kr)
    np.testing.assert_allclose(S.max(axis=2), oracle.chunk_scores(Qr, Kr), rtol=1e-14)
    for t in range(4):
        np.testing.assert_allclose(S[:, :, t], oracle.chunk_scores_loops(Qr[:, t:t + 1], Kr), rtol=1e-12)


def test_doc_score_argmax_ties_go_to_lowest_chunk_then_token():
    rng = np.random.default_rng(4)
    Qr, Kr, off = _route_case(rng, B=1, T=3, lens=(4,))
    for g in range(2):                # chunk 1 aligned with token 0, so the max sits there
        Kr[1, g] = Qr[0, 0, 2 * g] + Qr[0, 0, 2 * g + 1]
    Kr[2] = Kr[1]                     # chunks 1 and 2 equal
    Qr[0, 2] = Qr[0, 0]               # tokens 0 and 2 equal
    score, ac, at = bw.doc_score_argmax(Qr, Kr, off)
    s = np.array([[oracle.chunk_scores_loops(Qr[:, t:t + 1], Kr[n:n + 1])[0, 0] for t in range(3)]
                  for n in range(4)])
    assert s[1, 0] == s[1, 2] == s[2, 0] == s[2, 2] == s.max()
    assert (ac[0, 0], at[0, 0]) == (1, 0)


@pytest.mark.parametrize("G", [1, 2, 4])
def test_route_gradients_match_finite_differences(G):
    rng = np.random.default_rng(20 + G)
    Qr, Kr, off = _route_case(rng, Hq=4, Hkv=4 // G)
    dscore = rng.standard_normal((Qr.shape[0], len(off) - 1))
    # the arg max must be strict by a margin so the step does not cross it
    for b in range(Qr.shape[0]):
        for doc in range(len(off) - 1):
            vals = np.sort([oracle.chunk_scores_loops(Qr[b:b + 1, t:t + 1], Kr[n:n + 1])[0, 0]
                            for n in range(off[doc], off[doc + 1]) for t in range(Qr.shape[1])])
            assert len(vals) == 1 or vals[-1] - vals[-2] > 1e-4
    dQr, dKr = bw.route_score_bwd(Qr, Kr, off, dscore)
    loss = lambda: float(np.sum(dscore * bw.doc_score_argmax(Qr, Kr, off)[0]))
    np.testing.assert_allclose(dQr, _fd(loss, Qr, 1e-6), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dKr, _fd(loss, Kr, 1e-6), rtol=1e-6, atol=1e-8)


def test_route_gradients_are_orthogonal_to_their_vectors():
    # cos is invariant under q -> a q and k -> a k (a > 0), so <q, dq> = <k, dk> = 0
    rng = np.random.default_rng(9)
    Qr, Kr, off = _route_case(rng, B=3, T=5, Hq=8, Hkv=2, d=16, lens=(3, 5, 1, 2))
    dscore = rng.standard_normal((3, 4))
    dQr, dKr = bw.route_score_bwd(Qr, Kr, off, dscore)
    np.testing.assert_allclose(np.sum(Qr * dQr, axis=-1), 0.0, atol=1e-12)
    np.testing.assert_allclose(np.sum(Kr * dKr, axis=-1), 0.0, atol=1e-12)
    assert np.abs(dQr).max() > 1e-3 and np.abs(dKr).max() > 1e-3
    # only the arg-max token of each (query, document) receives a gradient
    _, _, at = bw.doc_score_argmax(Qr, Kr, off)
    for b in range(3):
        hit = set(at[b].tolist())
        for t in range(5):
            if t not in hit:
                assert np.all(dQr[b, t] == 0.0)


def test_route_gradient_of_a_zero_key_row():
    # below eps the key norm is the constant eps: d cos / dk = q / (|q| eps)
    # and d cos / dq = 0 (k = 0)
    rng = np.random.default_rng(1)
    Qr, Kr, off = _route_case(rng, B=1, T=1, Hq=2, Hkv=2, d=8, lens=(1,))
    Kr[0, 1] = 0.0
    dQr, dKr = bw.route_score_bwd(Qr, Kr, off, np.ones((1, 1)))
    q = Qr[0, 0, 1]
    np.testing.assert_allclose(dKr[0, 1], 0.5 * q / (np.linalg.norm(q) * oracle.EPS), rtol=1e-12)
    kq = Kr[0, 0] / np.linalg.norm(Kr[0, 0])
    q0 = Qr[0, 0, 0]
    cos0 = q0 @ kq / np.linalg.norm(q0)
    np.testing.assert_allclose(dQr[0, 0, 0], 0.5 * (kq - cos0 * q0 / np.linalg.norm(q0)) / np.linalg.norm(q0),
                               rtol=1e-10)
    np.testing.assert_allclose(dQr[0, 0, 1], 0.0, atol=0)


@pytest.mark.parametrize("chunk_len,lens", [(3, (5, 1, 7)), (1, (2, 3)), (4, (4, 8))])
def test_encode_pool_gradients_match_finite_differences(chunk_len, lens):
    rng = np.random.default_rng(40 + chunk_len)
    tok = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, H, d = int(tok[-1]), 2, 8
    K, V, Kr = (rng.standard_normal((T, H, d)) for _ in range(3))
    N = int(oracle.chunk_offsets(tok, chunk_len)[-1])
    gK, gV, gR = (rng.standard_normal((N, H, d)) for _ in range(3))
    dK, dV, dKr = bw.encode_pool_bwd(gK, gV, gR, tok, chunk_len, THETA)

    def loss():
        kb, vb, rb = oracle.encode_pool(K, V, Kr, tok, chunk_len, THETA)
        return float(np.sum(gK * kb) + np.sum(gV * vb) + np.sum(gR * rb))

    np.testing.assert_allclose(dK, _fd(loss, K), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dV, _fd(loss, V), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dKr, _fd(loss, Kr), rtol=1e-6, atol=1e-8)


def test_encode_pool_gradient_rows_sum_to_the_pooled_gradient():
    rng = np.random.default_rng(8)
    tok = np.array([0, 10, 13], dtype=np.int64)
    gK, gV, gR = (rng.standard_normal((5, 2, 8)) for _ in range(3))   # chunks 4: 3 + 2 = 5 rows
    dK, dV, dKr = bw.encode_pool_bwd(gK, gV, gR, tok, 4, THETA)
    off = oracle.chunk_offsets(tok, 4)
    for doc in range(2):
        s, e = tok[doc], tok[doc + 1]
        for c, r0 in enumerate(range(s, e, 4)):
            r1 = min(r0 + 4, e)
            np.testing.assert_allclose(dV[r0:r1].sum(axis=0), gV[off[doc] + c], rtol=1e-12)
            np.testing.assert_allclose(dKr[r0:r1].sum(axis=0), gR[off[doc] + c], rtol=1e-12)
            rot = oracle.rope(dK[r0:r1], (np.arange(r0, r1) - s)[:, None], THETA)   # back to rotated space
            np.testing.assert_allclose(rot.sum(axis=0), gK[off[doc] + c], rtol=1e-12, atol=1e-14)
