"""Pins of the oracle's stage 1 (document-wise RoPE + chunk mean pooling)."""

import math

import numpy as np
import pytest

import oracle


def _docs(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


def _inputs(T, H, d, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, H, d)), rng.standard_normal((T, H, d)),
            rng.standard_normal((T, H, d)))


def test_chunk_offsets_are_prefix_sums_of_ceil():
    assert oracle.chunk_offsets(_docs([5, 2, 7]), 2).tolist() == [0, 3, 4, 8]
    assert oracle.chunk_offsets(_docs([64, 65, 1]), 64).tolist() == [0, 1, 3, 4]


@pytest.mark.parametrize("c", [1, 2, 3, 4])
def test_matches_loop_form_ragged(c):
    lens = [5, 1, 7, 4]
    off = _docs(lens)
    K, V, Kr = _inputs(int(off[-1]), 2, 8)
    a = oracle.encode_pool(K, V, Kr, off, c, 1e4)
    b = oracle.encode_pool_loops(K, V, Kr, off, c, 1e4)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-12)


def test_v_and_kr_are_chunk_means():
    lens = [70, 64, 3, 129]
    off = _docs(lens)
    K, V, Kr = _inputs(int(off[-1]), 3, 16, seed=3)
    _, Vb, Rb = oracle.encode_pool(K, V, Kr, off, 64, 1e6)
    row = 0
    for doc in range(len(lens)):
        s, e = off[doc], off[doc + 1]
        for r0 in range(s, e, 64):
            r1 = min(r0 + 64, e)
            np.testing.assert_allclose(Vb[row], V[r0:r1].mean(axis=0), rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(Rb[row], Kr[r0:r1].mean(axis=0), rtol=1e-13, atol=1e-15)
            row += 1
    assert row == Vb.shape[0]


def test_chunk_len_one_is_rope_at_document_local_positions():
    lens = [3, 4, 2]
    off = _docs(lens)
    K, V, Kr = _inputs(int(off[-1]), 2, 8, seed=4)
    Kb, Vb, Rb = oracle.encode_pool(K, V, Kr, off, 1, 1e4)
    assert np.array_equal(Vb, V) and np.array_equal(Rb, Kr)
    for doc in range(3):
        s, e = off[doc], off[doc + 1]
        # first token of every document is at position 0: raw K, bit for bit
        assert np.array_equal(Kb[s], K[s])
        pos = np.arange(e - s)[:, None]
        np.testing.assert_allclose(Kb[s:e], oracle.rope(K[s:e], pos, 1e4), rtol=0, atol=0)


def test_positions_restart_per_document_moving_a_document_is_bitexact():
    rng = np.random.default_rng(6)
    lens = [9, 20, 5]
    docs = [rng.standard_normal((n, 2, 8)) for n in lens]
    perm = [2, 0, 1]

    def run(order):
        K = np.concatenate([docs[i] for i in order])
        off = _docs([lens[i] for i in order])
        Kb, _, _ = oracle.encode_pool(K, K, K, off, 4, 1e4)
        coff = oracle.chunk_offsets(off, 4)
        return {order[j]: Kb[coff[j]:coff[j + 1]] for j in range(len(order))}

    a, b = run([0, 1, 2]), run(perm)
    for i in range(3):
        assert np.array_equal(a[i], b[i])


def test_closed_form_two_token_chunk_d2():
    # d = 2, one document [x0, x1], chunk 2: Kbar = (x0 + R(1 rad) x1) / 2
    K = np.array([[[0.3, -1.2]], [[2.0, 0.5]]])
    Kb, Vb, _ = oracle.encode_pool(K, K, K, np.array([0, 2]), 2, 1e4)
    c, s = math.cos(1.0), math.sin(1.0)
    exp = [(0.3 + 2.0 * c - 0.5 * s) / 2, (-1.2 + 0.5 * c + 2.0 * s) / 2]
    np.testing.assert_allclose(Kb[0, 0], exp, atol=1e-15)
    np.testing.assert_allclose(Vb[0, 0], [(0.3 + 2.0) / 2, (-1.2 + 0.5) / 2], atol=1e-15)


def test_partial_last_chunk_is_mean_of_actual_rows():
    K, V, Kr = _inputs(5, 1, 4, seed=7)
    Kb, Vb, _ = oracle.encode_pool(K, V, Kr, np.array([0, 5]), 2, 1e4)
    assert Kb.shape[0] == 3
    np.testing.assert_allclose(Vb[2], V[4], atol=0)
    np.testing.assert_allclose(Kb[2], oracle.rope(K[4], 4, 1e4), atol=1e-15)


def test_rejects_empty_documents():
    K, V, Kr = _inputs(4, 1, 4)
    with pytest.raises(ValueError):
        oracle.encode_pool(K, V, Kr, np.array([0, 2, 2, 4]), 2, 1e4)


def test_chunk_mean_equals_pooled_v():
    lens = [70, 1, 130]
    off = _docs(lens)
    K, V, Kr = _inputs(int(off[-1]), 2, 8, seed=8)
    _, Vb, Rb = oracle.encode_pool(K, V, Kr, off, 64, 1e4)
    assert np.array_equal(oracle.chunk_mean(V, off, 64), Vb)
    assert np.array_equal(oracle.chunk_mean(Kr, off, 64), Rb)


def test_chunk_counts_are_ceilings():
    assert oracle.chunk_counts([1, 16, 17, 32, 33, 64], 16).tolist() == [1, 1, 2, 2, 3, 4]
    assert oracle.chunk_counts([5, 1, 7], 1).tolist() == [5, 1, 7]
