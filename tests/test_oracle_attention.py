"""Pins of the oracle's stage 3 (sparse attention with global RoPE offset)."""

import math

import numpy as np
import pytest
import torch

import oracle


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _case(rng, Tq=3, L=5, M=4, Hq=4, Hkv=2, d=8):
    return (_rand(rng, Tq, Hq, d), _rand(rng, M, Hkv, d), _rand(rng, M, Hkv, d),
            _rand(rng, L, Hkv, d), _rand(rng, L, Hkv, d))


def _one(Q, mK, mV, Kl, Vl, k, scale=None, theta=1e4):
    d = Q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    return oracle.sparse_attn(Q[None], mK, mV, [0, len(mK)], Kl[None], Vl[None], k, scale, theta)[0]


@pytest.mark.parametrize("Tq,L,M", [(1, 5, 3), (3, 5, 4), (5, 5, 0), (2, 6, 1)])
def test_matches_loop_form(Tq, L, M):
    rng = np.random.default_rng(Tq * 10 + L + M)
    Q, mK, mV, Kl, Vl = _case(rng, Tq, L, M)
    got = _one(Q, mK, mV, Kl, Vl, 4)
    ref = oracle.sparse_attn_loops(Q, mK, mV, Kl, Vl, 4, 1 / math.sqrt(8), 1e4)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def _sdpa(q, k, v, mask):
    """torch CPU scaled_dot_product_attention, float64, heads first."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).permute(1, 0, 2)[None]
    out = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=torch.from_numpy(mask)[None, None])
    return out[0].permute(1, 0, 2).numpy()


def test_no_memory_equals_textbook_causal_rope_attention_and_ignores_k():
    rng = np.random.default_rng(9)
    Tq, L, Hq, Hkv, d = 4, 9, 4, 2, 16
    Q, _, _, Kl, Vl = _case(rng, Tq, L, 0, Hq, Hkv, d)
    empty = np.zeros((0, Hkv, d))
    G = Hq // Hkv
    for k in [0, 16, 1000]:
        got = _one(Q, empty, empty, Kl, Vl, k)
        q = oracle.rope(Q, (k + L - Tq + np.arange(Tq))[:, None], 1e4)
        kk = oracle.rope(Kl, (k + np.arange(L))[:, None], 1e4)
        mask = np.arange(L)[None, :] <= (L - Tq) + np.arange(Tq)[:, None]
        ref = _sdpa(q, np.repeat(kk, G, axis=1), np.repeat(Vl, G, axis=1), mask)
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(got, _one(Q, empty, empty, Kl, Vl, 0), rtol=1e-10, atol=1e-12)


def test_chunk_one_all_documents_selected_is_full_attention_at_doc_local_positions():
    rng = np.random.default_rng(10)
    Hq, Hkv, d, Tq, L = 2, 1, 8, 2, 3
    lens = [3, 2, 4]
    off = np.concatenate([[0], np.cumsum(lens)])
    Kd, Vd = _rand(rng, off[-1], Hkv, d), _rand(rng, off[-1], Hkv, d)
    Kb, Vb, _ = oracle.encode_pool(Kd, Vd, Kd, off, 1, 1e4)
    Q, _, _, Kl, Vl = _case(rng, Tq, L, 0, Hq, Hkv, d)
    k = len(lens)
    got = _one(Q, Kb, Vb, Kl, Vl, k)
    # full attention: every document token at its document-local position,
    # then the local tokens at k + j, causal only inside the local part
    doc_pos = np.concatenate([np.arange(n) for n in lens])
    keys = np.concatenate([oracle.rope(Kd, doc_pos[:, None], 1e4),
                           oracle.rope(Kl, (k + np.arange(L))[:, None], 1e4)])
    vals = np.concatenate([Vd, Vl])
    q = oracle.rope(Q, (k + L - Tq + np.arange(Tq))[:, None], 1e4)
    mask = np.concatenate([np.ones((Tq, off[-1]), bool),
                           np.arange(L)[None, :] <= (L - Tq) + np.arange(Tq)[:, None]], axis=1)
    ref = _sdpa(q, np.repeat(keys, Hq, axis=1), np.repeat(vals, Hq, axis=1), mask)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_constant_values_give_that_constant():
    rng = np.random.default_rng(11)
    Q, mK, _, Kl, _ = _case(rng, 3, 6, 5)
    vec = rng.standard_normal(8)
    mV = np.broadcast_to(vec, (5, 2, 8)).copy()
    Vl = np.broadcast_to(vec, (6, 2, 8)).copy()
    got = _one(Q, mK, mV, Kl, Vl, 4)
    np.testing.assert_allclose(got, np.broadcast_to(vec, got.shape), rtol=1e-13, atol=1e-13)


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(12)
    Tq, L, M = 3, 6, 5
    _, mK, mV, Kl, Vl = _case(rng, Tq, L, M)
    Q = np.zeros((Tq, 4, 8))
    got = _one(Q, mK, mV, Kl, Vl, 4)
    for i in range(Tq):
        vis = (L - Tq) + i + 1
        for h in range(4):
            g = h // 2
            ref = np.concatenate([mV[:, g], Vl[:vis, g]]).mean(axis=0)
            np.testing.assert_allclose(got[i, h], ref, rtol=1e-13, atol=1e-14)


def test_future_local_tokens_are_invisible():
    rng = np.random.default_rng(13)
    Tq, L = 3, 6
    Q, mK, mV, Kl, Vl = _case(rng, Tq, L, 2)
    base = _one(Q, mK, mV, Kl, Vl, 4)
    Kl2, Vl2 = Kl.copy(), Vl.copy()
    Kl2[L - 1] += 50.0
    Vl2[L - 1] -= 50.0
    got = _one(Q, mK, mV, Kl2, Vl2, 4)
    assert np.array_equal(got[: Tq - 1], base[: Tq - 1])   # earlier query tokens unchanged
    assert not np.allclose(got[Tq - 1], base[Tq - 1])       # the last one sees it


def test_shifting_k_equals_rotating_memory_keys_back():
    rng = np.random.default_rng(14)
    Q, mK, mV, Kl, Vl = _case(rng, 2, 5, 6)
    for k, delta in [(4, 3), (16, 100), (0, 7)]:
        a = _one(Q, mK, mV, Kl, Vl, k + delta)
        b = _one(Q, oracle.rope(mK, np.full((6, 1), -delta), 1e4), mV, Kl, Vl, k)
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)
