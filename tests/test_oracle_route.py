"""Pins of the oracle's stage 2a (cosine routing, document max, top-k)."""

import math

import numpy as np
import pytest

import msa_synth
import oracle


def test_matches_scalar_loops():
    rng = np.random.default_rng(0)
    Qr = rng.standard_normal((2, 3, 4, 8))
    Kb = rng.standard_normal((5, 2, 8))
    np.testing.assert_allclose(oracle.chunk_scores(Qr, Kb), oracle.chunk_scores_loops(Qr, Kb),
                               rtol=1e-13, atol=1e-14)


def test_closed_form_single_head():
    for a in [0.0, 0.3, 1.0, 2.5, math.pi]:
        Qr = np.array([[[[2.0, 0.0]]]])
        Kb = np.array([[[3.0 * math.cos(a), 3.0 * math.sin(a)]]])
        assert abs(oracle.chunk_scores(Qr, Kb)[0, 0] - math.cos(a)) < 1e-15


def test_mean_of_head_cosines_not_cosine_of_mean_head():
    Qr = np.array([[[[1.0, 0.0], [0.0, 10.0]]]])      # two query heads
    Kb = np.array([[[1.0, 0.0]]])                     # one KV head
    assert abs(oracle.chunk_scores(Qr, Kb)[0, 0] - 0.5) < 1e-15


def test_gqa_maps_head_h_to_kv_head_h_div_g():
    e0, e1 = [1.0, 0.0], [0.0, 1.0]
    Qr = np.array([[[e0, e0, e1, e1]]])
    Kb = np.array([[e0, e1]])
    assert abs(oracle.chunk_scores(Qr, Kb)[0, 0] - 1.0) < 1e-15   # h % Hkv would give 0.5


def test_max_over_query_tokens():
    Qr = np.array([[[[1.0, 0.0]], [[-1.0, 0.0]], [[0.0, 1.0]]]])
    Kb = np.array([[[1.0, 0.0]]])
    assert oracle.chunk_scores(Qr, Kb)[0, 0] == 1.0


def test_zero_vector_scores_zero():
    Qr = np.zeros((1, 1, 2, 4))
    Kb = np.ones((3, 1, 4))
    assert np.array_equal(oracle.chunk_scores(Qr, Kb), np.zeros((1, 3)))


def test_power_of_two_scaling_is_bitexact():
    rng = np.random.default_rng(1)
    Qr = rng.standard_normal((1, 4, 8, 16))
    Kb = rng.standard_normal((30, 2, 16))
    base = oracle.chunk_scores(Qr, Kb)
    for p, q in [(3, -5), (-7, 9), (20, 0)]:
        assert np.array_equal(oracle.chunk_scores(Qr * 2.0 ** p, Kb * 2.0 ** q), base)


def test_permuting_chunks_permutes_scores():
    rng = np.random.default_rng(2)
    Qr = rng.standard_normal((2, 2, 4, 8))
    Kb = rng.standard_normal((17, 2, 8))
    perm = rng.permutation(17)
    assert np.array_equal(oracle.chunk_scores(Qr, Kb[perm]), oracle.chunk_scores(Qr, Kb)[:, perm])


def test_doc_scores_are_segment_maxima():
    c = np.array([[0.1, 0.5, -0.2, 0.3, 0.3, 0.9]])
    off = np.array([0, 2, 3, 6])
    assert oracle.doc_scores(c, off).tolist() == [[0.5, -0.2, 0.9]]


def test_topk_matches_textbook_stable_sort_exhaustively():
    rng = np.random.default_rng(3)
    for trial in range(200):
        n = int(rng.integers(1, 12))
        D = rng.integers(-3, 3, size=(1, n)).astype(np.float64)   # many ties
        ref = sorted(range(n), key=lambda i: -D[0, i])           # Python sort is stable
        for k in range(1, n + 1):
            ids, sc = oracle.topk_docs(D, k)
            assert ids[0].tolist() == ref[:k]
            assert sc[0].tolist() == [D[0, i] for i in ref[:k]]


def test_duplicate_document_ties_to_lowest_id():
    rng = np.random.default_rng(4)
    Qr = rng.standard_normal((1, 2, 4, 8))
    Kb = rng.standard_normal((6, 2, 8))
    Kb[4] = Kb[1]                             # doc 4 duplicates doc 1 (one chunk per doc)
    Qr[0, 0] = np.repeat(Kb[1], 2, axis=0)    # make doc 1 the best match
    off = np.arange(7)
    ids, sc, _, D = oracle.route(Qr, Kb, off, 2)
    assert D[0, 1] == D[0, 4]
    assert ids[0].tolist() == [1, 4]


def test_planted_documents_are_recovered():
    # the tiny fp32 workload: 64 docs x 256 tokens, chunk 16, Hq 4 / Hkv 2, d 64
    seed, Hq, Hkv, d, T, c = 0, 4, 2, 64, 32, 16
    lens = np.full(64, 256)
    off = msa_synth.prefix_offsets(lens)
    Kr = msa_synth.normal_f32(seed, 3, (int(off[-1]), Hkv, d)).astype(np.float64)
    Qr = msa_synth.normal_f32(seed, 4, (1, T, Hq, d)).astype(np.float64)
    planted = msa_synth.pick_planted(seed, 50, 64, 4)
    tok = np.random.default_rng(51).integers(0, T, size=4)
    for j, doc in enumerate(planted):
        Kr[off[doc]:off[doc + 1]] = msa_synth.planted_rows(seed, 60 + j, Qr[0, tok[j]], Hkv,
                                                           256, out="f32")
    _, _, Krb = oracle.encode_pool(Kr, Kr, Kr, off, c, 1e4)
    ids, sc, _, D = oracle.route(Qr, Krb, oracle.chunk_offsets(off, c), 4)
    assert sorted(ids[0].tolist()) == planted.tolist()
    others = np.delete(D[0], planted)
    assert sc[0].min() - others.max() >= 0.05
