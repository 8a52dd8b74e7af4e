"""HIP path vs the oracle, element by element, through the C ABI (GPU only).

Tolerances (stated where used):
  pooled rows      fp32 1e-5, bf16 2e-2, relative per (chunk, head) row:
                   |got - ref| <= rtol * (|ref| + rms(ref row))
  attention output fp32 1e-3, bf16 2e-2, max-abs of the normalised output
  chunk/doc scores 1e-4 absolute on the fp32-accumulating vector paths: a
                   score is (1/Hq) sum_g U_g . k_g/|k_g| with |U_g| <= G, and
                   a 128-term fp32 dot product errs by at most 128 * 2^-24 *
                   |U_g|, so the sum over Hkv groups / Hq errs by <= 8e-6;
                   rsqrt and the unit-query error add ~1e-6
                   3e-3 absolute on the matrix-core path (bf16, d 128,
                   B*Tq > 4), which rounds U to bf16 (relative 2^-9 per
                   element): |delta s| <= 2^-9
                   5e-3 absolute on the prefill GEMM path (Tq a multiple of
                   256 or at least 1,024), which also rounds the unit keys to
                   bf16: |delta s| <= 2^-9 + 2^-9 = 2^-8
  top-k            document id sets bit-exact on planted-margin inputs; on
                   unplanted inputs every selected id is a valid top-k under
                   the score tolerance and the order is (score desc, id asc)
"""

import math

import numpy as np
import pytest

import msa_synth
import oracle
from tests import peaked as P
from tests import workloads as W

pytestmark = pytest.mark.gpu

SCORE_TOL = 1e-4
# Matrix-core routing rounds the query group sums U to bf16 (relative 2^-9 per
# element); by Cauchy-Schwarz |delta s| <= (1/Hq) sum_g 2^-9 |U_g| <= 2^-9.
MFMA_SCORE_TOL = 3e-3
# The prefill GEMM path (Tq a multiple of 256, or at least 1,024 tokens) also
# rounds the unit keys K̄r/|K̄r| to bf16: |delta s| <= 2^-9 + 2^-9 = 2^-8 ~ 3.9e-3.
GEMM_SCORE_TOL = 5e-3


def _score_tol(dtype, d, B, Tq):
    if dtype != "bf16" or d != 128 or B * Tq <= 4:
        return SCORE_TOL                        # vector units
    if Tq > 1 and (Tq % 256 == 0 or Tq >= 1024):
        return GEMM_SCORE_TOL
    return MFMA_SCORE_TOL


@pytest.fixture(scope="module")
def torch_mod(gpu):
    import torch
    return torch


@pytest.fixture(scope="module")
def msa(gpu):
    import long_context_memory_chunk_amd as m
    m.lib()   # raises if the library is missing: no fallback
    return m


@pytest.fixture(scope="module")
def ctx128(msa):
    c = msa.msa_ctx_create(0, 128, 1e6, 16384)
    yield c
    c.close()


@pytest.fixture(scope="module")
def ctx64(msa):
    c = msa.msa_ctx_create(0, 64, 1e4, 4096)
    yield c
    c.close()


def _ctx(d, ctx64, ctx128):
    return ctx128 if d == 128 else ctx64


# ---------------------------------------------------------------- generator

def test_device_counter_fill_matches_numpy(torch_mod, msa):
    from msa_synth import device
    torch = torch_mod
    for seed, stream, start, count in [(0, 1, 0, 4096), (7, 3, 12345, 1000), (3, 1001, 2**33 + 8, 77)]:
        t = torch.empty(count, dtype=torch.bfloat16, device="cuda")
        device.fill_counter_bf16(t, seed, stream, start)
        torch.cuda.synchronize()
        assert np.array_equal(W.host_bits(t), msa_synth.counter_bf16(seed, stream, start, count))


# ---------------------------------------------------------------- stage 1

ENCODE_CASES = [
    # dtype, d, Hkv, chunk, lengths
    ("f32", 64, 2, 16, [256] * 6),
    ("f32", 128, 3, 5, [1, 7, 12, 3, 40]),
    ("bf16", 128, 8, 64, [128, 1024, 64, 65, 300, 999, 1]),
    ("bf16", 64, 4, 1, [3, 9, 1, 17]),
    ("bf16", 128, 8, 7, [50, 7, 8, 6, 2000]),
    ("bf16", 128, 1, 64, [4100]),
]


@pytest.mark.parametrize("dtype,d,Hkv,c,lens", ENCODE_CASES)
def test_encode_pool_parity(torch_mod, msa, ctx64, ctx128, dtype, d, Hkv, c, lens):
    torch = torch_mod
    ctx = _ctx(d, ctx64, ctx128)
    lens = np.array(lens, dtype=np.int64)
    tok = msa_synth.prefix_offsets(lens)
    coff = msa.msa_chunk_offsets(tok, c)
    assert np.array_equal(coff, oracle.chunk_offsets(tok, c))
    T, N = int(tok[-1]), int(coff[-1])
    K, V, Kr = (W.draw(21, s, (T, Hkv, d), dtype) for s in (1, 2, 3))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    KVbar = torch.full((N, 2, Hkv, d), float("nan"), dtype=tdt, device="cuda")
    Krbar = torch.full((N, Hkv, d), float("nan"), dtype=tdt, device="cuda")
    msa.msa_encode_pool(ctx, W.dev(K, dtype), W.dev(V, dtype), W.dev(Kr, dtype),
                        torch.from_numpy(tok).cuda(), torch.from_numpy(coff).cuda(), KVbar, Krbar, c,
                        int(lens.max()))
    torch.cuda.synchronize()
    Kb, Vb, Rb = oracle.encode_pool(W.widen(K, dtype), W.widen(V, dtype), W.widen(Kr, dtype), tok, c,
                                    ctx.rope_theta)
    kv = W.widen(W.host_bits(KVbar), dtype)
    kr = W.widen(W.host_bits(Krbar), dtype)
    rtol = 2e-2 if dtype == "bf16" else 1e-5
    assert W.rel_row_err(kv[:, 0], Kb) <= rtol
    assert W.rel_row_err(kv[:, 1], Vb) <= rtol
    assert W.rel_row_err(kr, Rb) <= rtol
    if dtype == "bf16":
        # tighter self-check: one rounding of an fp32 accumulation is within half a
        # bf16 ulp (<= 2^-8 relative) plus fp32 summation error
        for got, ref in ((kv[:, 0], Kb), (kv[:, 1], Vb), (kr, Rb)):
            assert W.rel_row_err(got, ref) <= 2 ** -8 + 1e-5


def _random_encode_cases(n, seed):
    """Seeded layouts: either dtype and head dim, 1-16 KV heads, chunk lengths
    1-64, and 1-40 documents whose lengths mix single tokens, lengths one off
    a chunk multiple and long documents (below the RoPE table of each head
    dim: 4096 positions for d = 64, 16384 for d = 128)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = ("bf16", "f32")[i % 2]
        d = (128, 128, 64)[i % 3]
        Hkv = int(rng.choice([1, 2, 3, 4, 8, 16]))
        c = int(rng.choice([1, int(rng.integers(2, 64)), 64]))
        lens = []
        for _ in range(int(rng.integers(1, 41))):
            kind = rng.integers(0, 4)
            if kind == 0:
                lens.append(1)
            elif kind == 1:
                lens.append(max(1, c * int(rng.integers(1, 9)) + int(rng.choice([-1, 0, 1]))))
            elif kind == 2:
                lens.append(int(rng.integers(2, 300)))
            else:
                lens.append(int(rng.integers(300, 4000 if d == 64 else 9000)))
        cases.append((dtype, d, Hkv, c, lens))
    return cases


@pytest.mark.parametrize("dtype,d,Hkv,c,lens", _random_encode_cases(10, 404))
def test_encode_pool_random_layouts(torch_mod, msa, ctx64, ctx128, dtype, d, Hkv, c, lens):
    test_encode_pool_parity(torch_mod, msa, ctx64, ctx128, dtype, d, Hkv, c, lens)


# ---------------------------------------------------------------- stage 2a

def _bank(dtype, N, Hkv, d, seed):
    if dtype == "bf16":
        return msa_synth.counter_bf16(seed, 77, 0, N * Hkv * d).reshape(N, Hkv, d)
    return msa_synth.normal_f32(seed, 77, (N, Hkv, d))


def _run_route(torch, msa, ctx, Qr_h, Kb_h, coff, top_k, dtype, Tq_override=None):
    B, Tq, Hq, d = Qr_h.shape
    N, Hkv, _ = Kb_h.shape
    n_docs = len(coff) - 1
    ws = msa.workspace(msa.msa_route_workspace_size(1 if dtype == "bf16" else 0, B, Tq, Hq, Hkv, N,
                                                    n_docs, top_k))
    ids = torch.empty((B, top_k), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, top_k), dtype=torch.float32, device="cuda")
    ch = torch.empty((B, N), dtype=torch.float32, device="cuda")
    dc = torch.empty((B, n_docs), dtype=torch.float32, device="cuda")
    msa.msa_route(ctx, W.dev(Qr_h, dtype), W.dev(Kb_h, dtype), torch.from_numpy(coff).cuda(), top_k,
                  ids, ws, out_scores=sc, out_chunk=ch, out_doc=dc)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), sc.cpu().numpy(), ch.cpu().numpy(), dc.cpu().numpy()


def _check_valid_topk(ids, sc, D_ref, tol):
    """ids/sc of one query against oracle doc scores: scores match, order is
    (score desc, id asc) on the returned scores, and no unselected document
    beats a selected one by more than the tolerance."""
    k = len(ids)
    assert len(set(ids.tolist())) == k
    np.testing.assert_allclose(sc, D_ref[ids], atol=tol, rtol=0)
    for a in range(k - 1):
        assert sc[a] > sc[a + 1] or (sc[a] == sc[a + 1] and ids[a] < ids[a + 1])
    kth = D_ref[ids].min()
    others = np.delete(D_ref, ids)
    if others.size:
        assert others.max() <= kth + 2 * tol


ROUTE_CASES = [
    # dtype, d, Hq, Hkv, B, Tq, n_docs, max chunks per doc, top_k
    ("bf16", 128, 32, 8, 1, 1, 300, 12, 16),     # decode scan, Qwen shape
    ("bf16", 128, 32, 8, 2, 2, 200, 9, 8),       # decode scan, 4 queries
    ("bf16", 128, 16, 4, 3, 1, 150, 5, 5),       # decode scan, 4 KV heads
    ("bf16", 128, 16, 16, 1, 1, 64, 3, 64),      # decode scan, 16 KV heads, k = 64
    ("bf16", 128, 32, 8, 1, 3, 100, 4, 7),       # 3 tokens of one query
    ("bf16", 128, 16, 8, 1, 1, 120, 6, 8),       # decode scan, G = 2 (half the head slots empty)
    ("bf16", 128, 24, 8, 2, 1, 110, 5, 6),       # decode scan, G = 3
    ("bf16", 128, 64, 8, 1, 2, 130, 7, 9),       # decode scan, G = 8 (two passes over the head slots)
    ("f32", 64, 4, 2, 1, 32, 64, 16, 4),         # tiny fp32 shape, generic scan
    ("bf16", 64, 8, 2, 2, 5, 90, 6, 10),         # generic scan
    ("bf16", 128, 32, 8, 3, 3, 120, 7, 9),       # 9 queries
    ("f32", 128, 8, 8, 1, 1, 10, 1, 10),         # k = n_docs
    ("bf16", 128, 32, 8, 32, 1, 300, 9, 16),     # matrix cores: 32 decode queries
    ("bf16", 128, 32, 8, 40, 1, 200, 5, 8),      # matrix cores: 40 queries, padded tile
    ("bf16", 128, 32, 8, 1, 256, 250, 8, 16),    # matrix cores: 256-token query, token max
    ("bf16", 128, 16, 4, 2, 128, 100, 12, 5),    # matrix cores: 4 KV heads, 2 queries
    ("bf16", 128, 16, 16, 6, 1, 90, 4, 7),       # matrix cores: 16 KV heads
    ("bf16", 128, 16, 4, 2, 512, 300, 6, 12),    # one GEMM: two 512-token queries, 4 KV heads
    # query lengths that are no multiple of a tile: padded rows left out of the token max
    ("bf16", 128, 32, 8, 1, 5, 200, 8, 16),      # 32-row tiles, 27 padded rows
    ("bf16", 128, 32, 8, 4, 2, 100, 4, 8),       # 32-row tiles, four 2-token queries
    ("bf16", 128, 16, 4, 3, 33, 100, 5, 9),      # 128-row tiles, 95 padded rows per query
    ("bf16", 128, 32, 8, 2, 100, 150, 6, 8),     # 128-row tiles, two queries
    ("bf16", 128, 32, 8, 1, 300, 200, 6, 16),    # three 128-row tiles, the last mostly padding
    ("bf16", 128, 32, 8, 2, 1100, 80, 5, 10),    # GEMM: two queries of five 256-row tiles each
    ("bf16", 128, 32, 8, 1, 1500, 80, 5, 10),    # GEMM, 36 padded rows
    ("bf16", 128, 32, 8, 1, 8000, 60, 5, 16),    # GEMM: an 8,000-token prompt
]


@pytest.mark.parametrize("dtype,d,Hq,Hkv,B,Tq,n_docs,maxc,k", ROUTE_CASES)
def test_route_parity_random(torch_mod, msa, ctx64, ctx128, dtype, d, Hq, Hkv, B, Tq, n_docs, maxc, k):
    ctx = _ctx(d, ctx64, ctx128)
    rng = np.random.default_rng(n_docs + Hq)
    counts = rng.integers(1, maxc + 1, size=n_docs)
    coff = msa_synth.prefix_offsets(counts)
    N = int(coff[-1])
    Kb = _bank(dtype, N, Hkv, d, 31)
    Qr = W.draw(32, 4, (B, Tq, Hq, d), dtype)
    ids, sc, ch, dc = _run_route(torch_mod, msa, ctx, Qr, Kb, coff, k, dtype)
    c_ref = oracle.chunk_scores(W.widen(Qr, dtype), W.widen(Kb, dtype))
    D_ref = oracle.doc_scores(c_ref, coff)
    tol = _score_tol(dtype, d, B, Tq)
    assert np.max(np.abs(ch - c_ref)) <= tol
    assert np.max(np.abs(dc - D_ref)) <= tol
    for b in range(B):
        _check_valid_topk(ids[b], sc[b], D_ref[b], tol)


def _random_route_cases(n, seed):
    """Seeded shapes cycling through the four chunk-score paths: the streaming
    scan (B*Tq <= 4), the matrix cores on a decode batch, 128- and 256-token
    query blocks (token tiles, the one-GEMM path), and query blocks of any
    length or head dim (generic scan, fp32 among them); KV heads 1-16, group
    sizes 1-8, ragged documents of 1-19 chunks, k up to 64."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        kind = i % 4
        Hkv = int(rng.choice([1, 2, 4, 8, 16]))
        G = int(rng.choice([1, 2, 4, 8]))
        dtype, d = "bf16", 128
        if kind == 0:
            B, Tq = int(rng.integers(1, 5)), 1
        elif kind == 1:
            B, Tq = int(rng.integers(5, 41)), 1
        elif kind == 2:
            B, Tq = int(rng.integers(1, 3)), int(rng.choice([128, 256]))
        else:
            B, Tq = int(rng.integers(1, 4)), int(rng.integers(2, 20))
            dtype = str(rng.choice(["bf16", "f32"]))
            d = int(rng.choice([64, 128]))
        n_docs = int(rng.integers(1, 400))
        k = int(rng.integers(1, min(n_docs, 64) + 1))
        cases.append((dtype, d, G * Hkv, Hkv, B, Tq, n_docs, int(rng.integers(1, 20)), k))
    return cases


@pytest.mark.parametrize("dtype,d,Hq,Hkv,B,Tq,n_docs,maxc,k", _random_route_cases(16, 502))
def test_route_parity_random_shapes(torch_mod, msa, ctx64, ctx128, dtype, d, Hq, Hkv, B, Tq, n_docs, maxc,
                                    k):
    test_route_parity_random(torch_mod, msa, ctx64, ctx128, dtype, d, Hq, Hkv, B, Tq, n_docs, maxc, k)


@pytest.mark.parametrize("Hkv,G,Tq", [(1, 4, 256), (2, 2, 512)])
def test_route_gemm_more_tiles_than_cus(torch_mod, msa, ctx128, Hkv, G, Tq):
    """The long-query GEMM over about 300 chunk tiles of 256 per query tile,
    more workgroups than the chip has CUs, so tiles of one XCD's super-tile
    run in several rounds; one KV head gives the shortest contraction (four
    32-wide stages: the copy pipeline's prologue and its last four stages
    with nothing in between)."""
    test_route_parity_random(torch_mod, msa, None, ctx128, "bf16", 128, G * Hkv, Hkv, 1, Tq, 6000, 25, 16)


@pytest.mark.parametrize("Tq", [5, 33, 100, 1100])
def test_route_padded_rows_stay_out_of_the_token_max(torch_mod, msa, ctx128, Tq):
    """Every real score is about -0.9 (keys point against the queries), so a
    padded query row -- zeros, score 0 -- that reached the token max would
    show as 0.  Tq 5 and 33 pad 32- and 128-row tiles, 100 a 128-row tile,
    1,100 the GEMM's 256-row tiles."""
    torch = torch_mod
    Hq, Hkv, d, k = 32, 8, 128, 8
    rng = np.random.default_rng(77)
    v = rng.standard_normal(d)
    Qr = v[None, None, None, :] + 0.1 * rng.standard_normal((1, Tq, Hq, d))
    counts = rng.integers(1, 5, size=60)
    coff = msa_synth.prefix_offsets(counts)
    N = int(coff[-1])
    Kb = -v[None, None, :] + 0.1 * rng.standard_normal((N, Hkv, d))
    Qr_b, Kb_b = oracle.f64_to_bf16_bits(Qr), oracle.f64_to_bf16_bits(Kb)
    ids, sc, ch, dc = _run_route(torch_mod, msa, ctx128, Qr_b, Kb_b, coff, k, "bf16")
    c_ref = oracle.chunk_scores(W.widen(Qr_b, "bf16"), W.widen(Kb_b, "bf16"))
    assert c_ref.max() < -0.5
    tol = _score_tol("bf16", d, 1, Tq)
    assert np.max(np.abs(ch - c_ref)) <= tol
    D_ref = oracle.doc_scores(c_ref, coff)
    assert np.max(np.abs(dc - D_ref)) <= tol
    _check_valid_topk(ids[0], sc[0], D_ref[0], tol)


@pytest.mark.parametrize("B,Tq", [(1, 1), (2, 1), (1, 16), (32, 1), (1, 256), (1, 200), (2, 77)])
def test_route_planted_exact_set(torch_mod, msa, ctx128, B, Tq):
    Hq, Hkv, d, k = 32, 8, 128, 16
    n_docs = max(500, 20 * B * k)
    counts = np.random.default_rng(3).integers(1, 10, size=n_docs)
    coff = msa_synth.prefix_offsets(counts)
    N = int(coff[-1])
    Kb = _bank("bf16", N, Hkv, d, 41)
    Qr = msa_synth.normal_bf16(42, 4, (B, Tq, Hq, d))
    qf = msa_synth.bf16_bits_to_f32(Qr)
    planted = []
    for b in range(B):
        pl = msa_synth.pick_planted(43 + b, 50, n_docs, k, exclude=[p for q in planted for p in q])
        planted.append(pl)
        toks = np.random.default_rng(44 + b).integers(0, Tq, size=k)
        for j, doc in enumerate(pl):
            Kb[coff[doc]:coff[doc + 1]] = msa_synth.planted_rows(45 + b, j, qf[b, toks[j]], Hkv,
                                                                 int(counts[doc]))
    ids, sc, ch, dc = _run_route(torch_mod, msa, ctx128, Qr, Kb, coff, k, "bf16")
    ids_ref, sc_ref, c_ref, D_ref = oracle.route(W.widen(Qr, "bf16"), W.widen(Kb, "bf16"), coff, k)
    for b in range(B):
        assert sorted(ids[b].tolist()) == sorted(planted[b].tolist())      # recovered
        assert sorted(ids[b].tolist()) == sorted(ids_ref[b].tolist())      # bit-exact set
        margin = sc_ref[b].min() - np.delete(D_ref[b], ids_ref[b]).max()
        assert margin >= 0.05
    assert np.max(np.abs(ch - c_ref)) <= _score_tol("bf16", d, B, Tq)


@pytest.mark.parametrize("dtype,d,Hq,Hkv,B,Tq", [
    ("bf16", 128, 32, 8, 1, 1),       # streaming scan
    ("bf16", 128, 32, 8, 32, 1),      # matrix cores, decode batch
    ("bf16", 128, 32, 8, 1, 256),     # prefill GEMM (normalised keys)
    ("f32", 64, 8, 2, 1, 4),          # generic scan
])
def test_route_zero_vectors(torch_mod, msa, ctx64, ctx128, dtype, d, Hq, Hkv, B, Tq):
    """A zero routing key (whole row or one KV head) and a zero query head give
    cosine 0 through max(|x|, eps), on every scan path."""
    ctx = _ctx(d, ctx64, ctx128)
    counts = np.random.default_rng(5).integers(1, 6, size=120)
    coff = msa_synth.prefix_offsets(counts)
    N = int(coff[-1])
    Kb = _bank(dtype, N, Hkv, d, 61).copy()
    Kb[::7] = 0                       # whole rows
    Kb[3::11, Hkv - 1] = 0            # the last KV head of other rows
    Qr = W.draw(62, 4, (B, Tq, Hq, d), dtype).copy()
    Qr[:, :, 1] = 0                   # one query head of every token
    ids, sc, ch, dc = _run_route(torch_mod, msa, ctx, Qr, Kb, coff, 8, dtype)
    c_ref = oracle.chunk_scores(W.widen(Qr, dtype), W.widen(Kb, dtype))
    D_ref = oracle.doc_scores(c_ref, coff)
    tol = _score_tol(dtype, d, B, Tq)
    assert np.all(np.isfinite(ch))
    assert np.max(np.abs(ch - c_ref)) <= tol
    assert np.max(np.abs(dc - D_ref)) <= tol
    for b in range(B):
        _check_valid_topk(ids[b], sc[b], D_ref[b], tol)


def test_route_single_document(torch_mod, msa, ctx128):
    """A bank of one document: top-1 is that document, scored by its best chunk."""
    Hq, Hkv, d = 32, 8, 128
    coff = np.array([0, 5], dtype=np.int64)
    Kb = _bank("bf16", 5, Hkv, d, 71)
    Qr = msa_synth.normal_bf16(72, 4, (1, 1, Hq, d))
    ids, sc, ch, dc = _run_route(torch_mod, msa, ctx128, Qr, Kb, coff, 1, "bf16")
    c_ref = oracle.chunk_scores(W.widen(Qr, "bf16"), W.widen(Kb, "bf16"))
    assert ids.tolist() == [[0]]
    assert abs(sc[0, 0] - c_ref[0].max()) <= _score_tol("bf16", d, 1, 1)


def test_route_ties_go_to_lowest_id(torch_mod, msa, ctx128):
    Hq, Hkv, d = 32, 8, 128
    counts = np.array([2, 3, 1, 2, 3, 2, 1, 4])
    coff = msa_synth.prefix_offsets(counts)
    N = int(coff[-1])
    Kb = _bank("bf16", N, Hkv, d, 51)
    # every chunk of docs 1, 4 and 6 is a copy of one row, and the query points at it
    row = Kb[coff[1]].copy()
    Qr = np.stack([row[h // (Hq // Hkv)] for h in range(Hq)])[None, None]
    for doc in (1, 4, 6):
        Kb[coff[doc]:coff[doc + 1]] = row
    ids, sc, _, dc = _run_route(torch_mod, msa, ctx128, Qr, Kb, coff, 3, "bf16")
    assert dc[0, 1] == dc[0, 4] == dc[0, 6]
    assert ids[0].tolist() == [1, 4, 6]


def test_route_long_document_spans(torch_mod, msa, ctx128):
    """A wave of 256 documents spanning more chunks than the document-start
    marks cover (256 x 150 chunks) finds documents by binary search; the next
    wave uses the marks.  16 planted documents over both waves come back."""
    Hq, Hkv, d, k = 32, 8, 128, 16
    counts = np.concatenate([np.full(256, 150), np.random.default_rng(71).integers(1, 20, size=44)])
    coff = msa_synth.prefix_offsets(counts)
    N = int(coff[-1])
    Kb = _bank("bf16", N, Hkv, d, 72)
    Qr = msa_synth.normal_bf16(73, 4, (1, 1, Hq, d))
    q = msa_synth.bf16_bits_to_f32(Qr)[0, 0]
    planted = np.array([0, 3, 77, 128, 200, 254, 255, 256, 257, 260, 270, 280, 290, 297, 298, 299])
    for j, doc in enumerate(planted):
        Kb[coff[doc]:coff[doc + 1]] = msa_synth.planted_rows(74, 100 + j, q, Hkv, int(counts[doc]))
    ids, sc, ch, dc = _run_route(torch_mod, msa, ctx128, Qr, Kb, coff, k, "bf16")
    ids_ref, sc_ref, c_ref, D_ref = oracle.route(W.widen(Qr, "bf16"), W.widen(Kb, "bf16"), coff, k)
    assert sorted(ids[0].tolist()) == sorted(ids_ref[0].tolist()) == planted.tolist()
    assert np.max(np.abs(dc - D_ref)) <= SCORE_TOL


def test_route_many_qualifying_candidates(torch_mod, msa, ctx128):
    """25,600 one-chunk documents: wave 0 holds 16 documents at cosine ~0.8 and
    waves 1..99 hold 15 documents each on the query's own direction (bit-
    identical rows, so their scores tie exactly).  Every wave list's 16th key
    is then at most wave 0's, and ~1,500 candidates reach that threshold: the
    final selection takes its full-merge path.  Ties go to the lowest ids."""
    Hq, Hkv, d, k = 32, 8, 128, 16
    n_docs = 25600
    coff = np.arange(n_docs + 1, dtype=np.int64)
    Kb = _bank("bf16", n_docs, Hkv, d, 81)
    hi = msa_synth.normal_bf16(82, 1, (Hkv, d))
    Qr = np.stack([hi[h // (Hq // Hkv)] for h in range(Hq)])[None, None]
    mid_f = 0.8 * msa_synth.bf16_bits_to_f32(hi) + 0.6 * msa_synth.normal_f32(82, 2, (Hkv, d))
    mid = msa_synth.f32_to_bf16_bits(mid_f)
    for doc in range(10, 26):
        Kb[doc] = mid
    for w in range(1, 100):
        for doc in range(256 * w + 5, 256 * w + 20):
            Kb[doc] = hi
    ids, sc, ch, dc = _run_route(torch_mod, msa, ctx128, Qr, Kb, coff, k, "bf16")
    ids_ref, sc_ref, c_ref, D_ref = oracle.route(W.widen(Qr, "bf16"), W.widen(Kb, "bf16"), coff, k)
    expect = list(range(261, 276)) + [517]
    assert ids[0].tolist() == ids_ref[0].tolist() == expect


def test_route_is_deterministic(torch_mod, msa, ctx128):
    counts = np.random.default_rng(5).integers(1, 9, size=400)
    coff = msa_synth.prefix_offsets(counts)
    Kb = _bank("bf16", int(coff[-1]), 8, 128, 61)
    Qr = msa_synth.normal_bf16(62, 4, (1, 1, 32, 128))
    a = _run_route(torch_mod, msa, ctx128, Qr, Kb, coff, 16, "bf16")
    b = _run_route(torch_mod, msa, ctx128, Qr, Kb, coff, 16, "bf16")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("B,Tq", [(1, 1), (3, 1), (8, 1), (2, 5), (1, 256)])
def test_route_query_not_16_byte_aligned(torch_mod, msa, ctx128, B, Tq):
    """A query tensor that starts 2 bytes past a 16-byte boundary (a view one
    element into a buffer): the operand prep takes its element-wise form on the
    streaming scan (B*Tq <= 4), the matrix cores (decode batch, short blocks)
    and the token-tile GEMM alike, with the same chunk scores and selection as
    the oracle (neo-ai.one MSA article, 全体設計 › アーキテクチャ, Fig. 2: cosine,
    head mean, token max, top-k)."""
    torch = torch_mod
    Hq, Hkv, d, k = 32, 8, 128, 12
    counts = np.random.default_rng(B * 100 + Tq).integers(1, 11, size=180)
    coff = msa_synth.prefix_offsets(counts)
    N = int(coff[-1])
    Kb = _bank("bf16", N, Hkv, d, 63)
    Qr = msa_synth.normal_bf16(64 + B, Tq, (B, Tq, Hq, d))
    flat = torch.empty(Qr.size + 1, dtype=torch.bfloat16, device="cuda")
    flat[1:].copy_(W.dev_bf16(Qr.reshape(-1)))
    Qd = flat[1:].view(B, Tq, Hq, d)
    assert Qd.data_ptr() % 16 == 2
    ws = msa.workspace(msa.msa_route_workspace_size(1, B, Tq, Hq, Hkv, N, len(coff) - 1, k))
    ids = torch.empty((B, k), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, k), dtype=torch.float32, device="cuda")
    ch = torch.empty((B, N), dtype=torch.float32, device="cuda")
    dc = torch.empty((B, len(coff) - 1), dtype=torch.float32, device="cuda")
    msa.msa_route(ctx128, Qd, W.dev_bf16(Kb), torch.from_numpy(coff).cuda(), k, ids, ws, out_scores=sc,
                  out_chunk=ch, out_doc=dc)
    torch.cuda.synchronize()
    ids, sc, ch, dc = ids.cpu().numpy(), sc.cpu().numpy(), ch.cpu().numpy(), dc.cpu().numpy()
    c_ref = oracle.chunk_scores(W.widen(Qr, "bf16"), W.widen(Kb, "bf16"))
    D_ref = oracle.doc_scores(c_ref, coff)
    tol = _score_tol("bf16", d, B, Tq)
    assert np.max(np.abs(ch - c_ref)) <= tol
    assert np.max(np.abs(dc - D_ref)) <= tol
    for b in range(B):
        _check_valid_topk(ids[b], sc[b], D_ref[b], tol)
    # the aligned call on the same values: the same chunk scores within the path's tolerance
    _, _, ch_a, _ = _run_route(torch, msa, ctx128, Qr, Kb, coff, k, "bf16")
    assert np.max(np.abs(ch - ch_a)) <= tol


# ---------------------------------------------------------------- stage 2b

def test_gather_matches_oracle_indexing(torch_mod, msa):
    torch = torch_mod
    Hkv, d, n_docs = 8, 128, 50
    counts = np.random.default_rng(7).integers(1, 12, size=n_docs)
    coff = msa_synth.prefix_offsets(counts)
    N = int(coff[-1])
    bank = msa_synth.counter_bf16(3, 5, 0, N * 2 * Hkv * d).reshape(N, 2, Hkv, d)
    host = torch.empty((N, 2, Hkv, d), dtype=torch.bfloat16, pin_memory=True)
    host.copy_(W.dev_bf16(bank, "cpu"))
    ids = np.array([[7, 3, 8, 9, 40], [0, 49, 12, 13, 1]], dtype=np.int32)   # adjacent runs merge
    cap = 200
    dst = torch.zeros((cap, 2, Hkv, d), dtype=torch.bfloat16, device="cuda")
    mo_host = torch.zeros(3, dtype=torch.int64, pin_memory=True)
    mo_dev = torch.zeros(3, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    msa.msa_gather(host, 2 * Hkv * d * 2, N, coff, ids, 5, dst, cap, mo_host, mo_dev, side=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    mo = mo_host.numpy()
    assert np.array_equal(mo_dev.cpu().numpy(), mo)
    got = W.host_bits(dst)
    for b in range(2):
        ref, m = oracle.gather_rows(bank, coff, ids[b])
        assert mo[b + 1] - mo[b] == m
        assert np.array_equal(got[mo[b]:mo[b + 1]], ref)


def test_gather_rejects_overflow_and_duplicates(torch_mod, msa):
    torch = torch_mod
    coff = np.array([0, 4, 8, 12], dtype=np.int64)
    host = torch.zeros((12, 64), dtype=torch.uint8, pin_memory=True)
    dst = torch.zeros((12, 64), dtype=torch.uint8, device="cuda")
    mo = torch.zeros(2, dtype=torch.int64, pin_memory=True)
    with pytest.raises(msa.MsaError, match="cap_rows"):
        msa.msa_gather(host, 64, 12, coff, np.array([[0, 2]], np.int32), 2, dst, 7, mo)
    with pytest.raises(msa.MsaError, match="twice"):
        msa.msa_gather(host, 64, 12, coff, np.array([[1, 1]], np.int32), 2, dst, 12, mo)
    with pytest.raises(msa.MsaError, match="outside"):
        msa.msa_gather(host, 64, 12, coff, np.array([[1, 3]], np.int32), 2, dst, 12, mo)


# ---------------------------------------------------------------- stage 3

ATTN_CASES = [
    # dtype, d, Hq, Hkv, B, Tq, L, rows per query, q_offset
    ("f32", 64, 4, 2, 1, 32, 32, [64], 4),            # tiny fp32 shape
    ("bf16", 128, 32, 8, 1, 1, 257, [152], 16),       # decode, Qwen shape
    ("bf16", 128, 32, 8, 1, 1, 2048, [125], 16),      # decode, 2K local
    ("bf16", 128, 32, 8, 3, 4, 300, [30, 0, 700], 16),  # ragged memory, one empty
    ("bf16", 64, 8, 8, 2, 5, 5, [3, 9], 2),           # G = 1, Tq = L
    ("f32", 128, 16, 1, 1, 7, 19, [260], 33),         # G = 16, several splits
    ("bf16", 128, 32, 8, 1, 64, 600, [250], 32),      # short prefill (matrix cores)
    ("bf16", 128, 32, 8, 1, 256, 256, [152], 16),     # prefill, Tq = L (matrix cores)
    ("bf16", 128, 32, 8, 2, 200, 500, [0, 300], 16),  # partial query tile, one query without memory
    ("bf16", 128, 8, 8, 1, 130, 130, [70], 8),        # G = 1, ragged tile
    ("bf16", 128, 16, 1, 1, 96, 1000, [64], 16),      # G = 16
    ("bf16", 128, 64, 8, 2, 1, 700, [90, 200], 16),   # G = 8 decode
    ("bf16", 128, 32, 8, 4, 1, 8192, [500, 0, 1000, 37], 16),  # several 64-key chunks per workgroup
    ("bf16", 128, 32, 8, 2, 1, 1, [0, 5], 16),        # one local key; one query sees only it
    ("bf16", 128, 8, 8, 2, 1, 400, [37, 130], 16),    # decode, G = 1
    ("bf16", 128, 16, 8, 3, 2, 333, [64, 95, 1], 16), # G = 2, two tokens, blocks across the memory end
    ("bf16", 128, 32, 8, 2, 63, 700, [300, 129], 16), # 63 tokens: the longest query on the decode kernel
    ("bf16", 128, 64, 8, 3, 3, 2000, [1000, 31, 0], 16),  # G = 8, several chunks per workgroup
    ("f32", 64, 4, 2, 2, 1, 1, [0, 3], 4),            # the same on the generic kernel
]


@pytest.mark.parametrize("dtype,d,Hq,Hkv,B,Tq,L,rows,qoff", ATTN_CASES)
def test_sparse_attn_parity(torch_mod, msa, ctx64, ctx128, dtype, d, Hq, Hkv, B, Tq, L, rows, qoff):
    torch = torch_mod
    ctx = _ctx(d, ctx64, ctx128)
    mem_off = msa_synth.prefix_offsets(rows)
    M = int(mem_off[-1])
    Q = W.draw(71, 1, (B, Tq, Hq, d), dtype)
    KV = W.draw(71, 2, (max(M, 1), 2, Hkv, d), dtype)
    Kl = W.draw(71, 3, (B, L, Hkv, d), dtype)
    Vl = W.draw(71, 4, (B, L, Hkv, d), dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    O = torch.full((B, Tq, Hq, d), float("nan"), dtype=tdt, device="cuda")
    ws = msa.workspace(msa.msa_sparse_attn_workspace_size(1 if dtype == "bf16" else 0, B, Tq, Hq, Hkv,
                                                          max(rows), L))
    msa.msa_sparse_attn(ctx, W.dev(Q, dtype), W.dev(KV, dtype), torch.from_numpy(mem_off).cuda(),
                        max(rows), W.dev(Kl, dtype), W.dev(Vl, dtype), qoff, W.scale_of(d), O, ws)
    torch.cuda.synchronize()
    kv = W.widen(KV, dtype)
    ref = oracle.sparse_attn(W.widen(Q, dtype), kv[:, 0], kv[:, 1], mem_off, W.widen(Kl, dtype),
                             W.widen(Vl, dtype), qoff, W.scale_of(d), ctx.rope_theta)
    got = W.widen(W.host_bits(O), dtype)
    tol = 2e-2 if dtype == "bf16" else 1e-3
    P.assert_attn_close(got, ref, tol, f"{dtype} d={d} G={Hq // Hkv} B={B} Tq={Tq} L={L} rows={rows}")


def _random_attn_cases(n, seed):
    """Seeded shapes for the decode / short-query kernel: G in {1, 2, 4, 8},
    1-5 query tokens, ragged memory rows (some queries without any), local
    lengths from Tq to 700 and offsets k, so blocks start on every alignment
    against the memory/local boundary and the end."""
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        G = (1, 2, 4, 8)[k % 4]
        Hkv = int(rng.choice([1, 2, 8]))
        B = int(rng.integers(1, 5))
        Tq = int(rng.integers(1, 6))
        L = int(rng.integers(Tq, 701))
        rows = [int(r) if rng.random() > 0.2 else 0 for r in rng.integers(0, 500, size=B)]
        qoff = int(rng.integers(0, 64))
        cases.append((G * Hkv, Hkv, B, Tq, L, rows, qoff))
    return cases


@pytest.mark.parametrize("Hq,Hkv,B,Tq,L,rows,qoff", _random_attn_cases(12, 2024))
def test_sparse_attn_random_decode_shapes(torch_mod, msa, ctx128, Hq, Hkv, B, Tq, L, rows, qoff):
    torch = torch_mod
    d = 128
    mem_off = msa_synth.prefix_offsets(rows)
    M = int(mem_off[-1])
    Q = W.draw(91, 1, (B, Tq, Hq, d), "bf16")
    KV = W.draw(91, 2, (max(M, 1), 2, Hkv, d), "bf16")
    Kl = W.draw(91, 3, (B, L, Hkv, d), "bf16")
    Vl = W.draw(91, 4, (B, L, Hkv, d), "bf16")
    O = torch.full((B, Tq, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = msa.workspace(msa.msa_sparse_attn_workspace_size(1, B, Tq, Hq, Hkv, max(max(rows), 1), L))
    msa.msa_sparse_attn(ctx128, W.dev(Q, "bf16"), W.dev(KV, "bf16"), torch.from_numpy(mem_off).cuda(),
                        max(max(rows), 1), W.dev(Kl, "bf16"), W.dev(Vl, "bf16"), qoff, W.scale_of(d), O, ws)
    torch.cuda.synchronize()
    kv = W.widen(KV, "bf16")
    ref = oracle.sparse_attn(W.widen(Q, "bf16"), kv[:, 0], kv[:, 1], mem_off, W.widen(Kl, "bf16"),
                             W.widen(Vl, "bf16"), qoff, W.scale_of(d), ctx128.rope_theta)
    got = W.widen(W.host_bits(O), "bf16")
    P.assert_attn_close(got, ref, 2e-2, f"G={Hq // Hkv} B={B} Tq={Tq} L={L} rows={rows} k={qoff}")


def test_sparse_attn_is_deterministic(torch_mod, msa, ctx128):
    torch = torch_mod
    Q = W.dev_bf16(msa_synth.normal_bf16(81, 1, (1, 1, 32, 128)))
    KV = W.dev_bf16(msa_synth.normal_bf16(81, 2, (300, 2, 8, 128)))
    Kl = W.dev_bf16(msa_synth.normal_bf16(81, 3, (1, 1000, 8, 128)))
    Vl = W.dev_bf16(msa_synth.normal_bf16(81, 4, (1, 1000, 8, 128)))
    mo = torch.tensor([0, 300], dtype=torch.int64, device="cuda")
    ws = msa.workspace(msa.msa_sparse_attn_workspace_size(1, 1, 1, 32, 8, 300, 1000))
    outs = []
    for _ in range(2):
        O = torch.empty((1, 1, 32, 128), dtype=torch.bfloat16, device="cuda")
        msa.msa_sparse_attn(ctx128, Q, KV, mo, 300, Kl, Vl, 16, W.scale_of(128), O, ws)
        outs.append(W.host_bits(O))
    assert np.array_equal(outs[0], outs[1])


def test_sparse_attn_running_max_rises_every_block(torch_mod, msa, ctx128):
    """Memory keys whose scores grow by far more than the lazy-rescale margin
    from one 32-key block to the next (K row r of KV head g is 0.5 r times the
    unit direction of query head g G, rotated at the query's position), so the
    running max of every head is raised, and the output accumulated so far
    rescaled, block after block."""
    torch = torch_mod
    Hq, Hkv, d, L, qoff, rows = 32, 8, 128, 40, 16, 600
    G = Hq // Hkv
    Q = W.draw(83, 1, (1, 1, Hq, d), "bf16")
    q = W.widen(Q, "bf16")[0, 0]
    rq = oracle.rope(q, np.full(Hq, qoff + L - 1), ctx128.rope_theta)
    unit = rq / np.linalg.norm(rq, axis=-1, keepdims=True)
    kv = np.empty((rows, 2, Hkv, d))
    kv[:, 0] = 0.5 * np.arange(rows, dtype=np.float64)[:, None, None] * unit[::G][None]
    kv[:, 1] = W.widen(W.draw(83, 2, (rows, Hkv, d), "bf16"), "bf16")
    KV = oracle.f64_to_bf16_bits(kv)
    Kl = W.draw(83, 3, (1, L, Hkv, d), "bf16")
    Vl = W.draw(83, 4, (1, L, Hkv, d), "bf16")
    mem_off = np.array([0, rows], dtype=np.int64)
    O = torch.full((1, 1, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = msa.workspace(msa.msa_sparse_attn_workspace_size(1, 1, 1, Hq, Hkv, rows, L))
    msa.msa_sparse_attn(ctx128, W.dev(Q, "bf16"), W.dev(KV, "bf16"), torch.from_numpy(mem_off).cuda(), rows,
                        W.dev(Kl, "bf16"), W.dev(Vl, "bf16"), qoff, W.scale_of(d), O, ws)
    torch.cuda.synchronize()
    kvw = W.widen(KV, "bf16")
    ref = oracle.sparse_attn(q[None, None], kvw[:, 0], kvw[:, 1], mem_off, W.widen(Kl, "bf16"),
                             W.widen(Vl, "bf16"), qoff, W.scale_of(d), ctx128.rope_theta)
    got = W.widen(W.host_bits(O), "bf16")
    P.assert_attn_close(got, ref, 2e-2, "rising running max")


# ---------------------------------------------------------------- validation with a context

def test_encode_rejects_documents_longer_than_the_rope_table(torch_mod, msa, ctx64):
    """ctx64 has max_pos 4096: a document of 4,097 tokens needs position 4096,
    so both encode calls refuse it before enqueueing anything; 4,096 tokens
    is the longest accepted."""
    torch = torch_mod
    for n in (4097, 4096):
        lens = np.array([3, n], dtype=np.int64)
        tok = msa_synth.prefix_offsets(lens)
        coff, longest = msa.msa_chunk_offsets(tok, 16, with_max_len=True)
        assert longest == n
        T, N = int(tok[-1]), int(coff[-1])
        X = torch.zeros((T, 2, 64), dtype=torch.float32, device="cuda")
        KVbar = torch.zeros((N, 2, 2, 64), dtype=torch.float32, device="cuda")
        Krbar = torch.zeros((N, 2, 64), dtype=torch.float32, device="cuda")
        tok_d, coff_d = torch.from_numpy(tok).cuda(), torch.from_numpy(coff).cuda()
        if n > ctx64.max_pos:
            with pytest.raises(msa.MsaError) as e:
                msa.msa_encode_pool(ctx64, X, X, X, tok_d, coff_d, KVbar, Krbar, 16, longest)
            assert e.value.status == msa.MSA_ERR_INVALID_ARG and "max_pos" in str(e.value)
            with pytest.raises(msa.MsaError) as e:
                msa.msa_encode_pool_bwd(ctx64, KVbar, Krbar, tok_d, coff_d, X, X, X, 16, longest)
            assert e.value.status == msa.MSA_ERR_INVALID_ARG and "max_pos" in str(e.value)
        else:
            msa.msa_encode_pool(ctx64, X, X, X, tok_d, coff_d, KVbar, Krbar, 16, longest)
            torch.cuda.synchronize()
            assert bool(torch.isfinite(KVbar).all())


def test_encode_marks_a_document_longer_than_max_doc_len_with_nan(torch_mod, msa, ctx128):
    """A max_doc_len below a document's real length is a caller error the
    host cannot see (the offsets are on the device): that document's pooled
    rows (and its token gradients in the backward) come out NaN, the other
    documents' rows are exact, and nothing reads past the RoPE table."""
    torch = torch_mod
    lens = np.array([40, 100, 17], dtype=np.int64)
    tok = msa_synth.prefix_offsets(lens)
    coff = msa.msa_chunk_offsets(tok, 16)
    T, N = int(tok[-1]), int(coff[-1])
    K, V, Kr = (W.draw(23, s, (T, 2, 128), "f32") for s in (1, 2, 3))
    KVbar = torch.zeros((N, 2, 2, 128), dtype=torch.float32, device="cuda")
    Krbar = torch.zeros((N, 2, 128), dtype=torch.float32, device="cuda")
    tok_d, coff_d = torch.from_numpy(tok).cuda(), torch.from_numpy(coff).cuda()
    msa.msa_encode_pool(ctx128, W.dev_f32(K), W.dev_f32(V), W.dev_f32(Kr), tok_d, coff_d, KVbar, Krbar, 16, 50)
    dK = torch.zeros((T, 2, 128), dtype=torch.float32, device="cuda")
    dV, dKr = torch.zeros_like(dK), torch.zeros_like(dK)
    msa.msa_encode_pool_bwd(ctx128, KVbar, Krbar, tok_d, coff_d, dK, dV, dKr, 16, 50)
    torch.cuda.synchronize()
    kv, kr = KVbar.cpu().numpy(), Krbar.cpu().numpy()
    long_rows = slice(int(coff[1]), int(coff[2]))
    assert np.all(np.isnan(kv[long_rows])) and np.all(np.isnan(kr[long_rows]))
    Kb, Vb, Rb = oracle.encode_pool(W.widen(K, "f32"), W.widen(V, "f32"), W.widen(Kr, "f32"), tok, 16,
                                    ctx128.rope_theta)
    for rows in (slice(int(coff[0]), int(coff[1])), slice(int(coff[2]), int(coff[3]))):
        assert W.rel_row_err(kv[rows, 0], Kb[rows]) <= 1e-5
        assert W.rel_row_err(kv[rows, 1], Vb[rows]) <= 1e-5
        assert W.rel_row_err(kr[rows], Rb[rows]) <= 1e-5
    toks = slice(int(tok[1]), int(tok[2]))
    for g in (dK, dV, dKr):
        g = g.cpu().numpy()
        assert np.all(np.isnan(g[toks]))
        assert np.all(np.isfinite(g[:int(tok[1])])) and np.all(np.isfinite(g[int(tok[2]):]))


def test_validation_errors_enqueue_nothing(torch_mod, msa, ctx128):
    torch = torch_mod
    Qr = torch.zeros((1, 1, 30, 128), dtype=torch.bfloat16, device="cuda")
    Kb = torch.zeros((10, 8, 128), dtype=torch.bfloat16, device="cuda")
    coff = torch.arange(11, dtype=torch.int64, device="cuda")
    ids = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    ws = msa.workspace(1 << 20)
    with pytest.raises(msa.MsaError) as e:                       # Hq % Hkv
        msa.msa_route(ctx128, Qr, Kb, coff, 4, ids, ws)
    assert e.value.status == msa.MSA_ERR_INVALID_ARG
    Qr = torch.zeros((1, 1, 32, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(msa.MsaError):                            # top_k > n_docs
        msa.msa_route(ctx128, Qr, Kb, coff, 11, torch.zeros((1, 11), dtype=torch.int32, device="cuda"), ws)
    with pytest.raises(msa.MsaError) as e:                       # small workspace
        msa.msa_route(ctx128, Qr, Kb, coff, 4, ids, msa.workspace(256)[:16])
    assert e.value.status == msa.MSA_ERR_WORKSPACE
    Q = torch.zeros((1, 1, 24, 128), dtype=torch.bfloat16, device="cuda")
    Kl = torch.zeros((1, 8, 8, 128), dtype=torch.bfloat16, device="cuda")
    O = torch.zeros_like(Q)
    with pytest.raises(msa.MsaError) as e:                       # G = 3 unsupported
        msa.msa_sparse_attn(ctx128, Q, None, torch.zeros(2, dtype=torch.int64, device="cuda"), 0,
                            Kl, Kl, 0, 0.1, O, ws)
    assert e.value.status == msa.MSA_ERR_INVALID_ARG or e.value.status == msa.MSA_ERR_UNSUPPORTED
    Q = torch.zeros((1, 1, 32, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(msa.MsaError, match="max_pos"):           # positions beyond the table
        msa.msa_sparse_attn(ctx128, Q, None, torch.zeros(2, dtype=torch.int64, device="cuda"), 0,
                            Kl, Kl, 16380, 0.1, torch.zeros_like(Q), ws)
    torch.cuda.synchronize()


def test_gather_device_matches_oracle_and_host_gather(torch_mod, msa, ctx128):
    torch = torch_mod
    Hkv, d, n_docs = 8, 128, 60
    counts = np.random.default_rng(17).integers(1, 12, size=n_docs)
    coff = msa_synth.prefix_offsets(counts)
    N = int(coff[-1])
    bank = msa_synth.counter_bf16(4, 6, 0, N * 2 * Hkv * d).reshape(N, 2, Hkv, d)
    host = torch.empty((N, 2, Hkv, d), dtype=torch.bfloat16, pin_memory=True)
    host.copy_(W.dev_bf16(bank, "cpu"))
    ids = np.array([[7, 3, 8, 9, 40], [0, 59, 12, 13, 1], [30, 31, 32, 33, 34]], dtype=np.int32)
    B, k = ids.shape
    cap = int(sum(np.diff(coff)[ids[b]].sum() for b in range(B)))
    row_bytes = 2 * Hkv * d * 2
    coff_dev = torch.from_numpy(coff).cuda()
    dst = torch.zeros((cap, 2, Hkv, d), dtype=torch.bfloat16, device="cuda")
    mo = torch.zeros(B + 1, dtype=torch.int64, device="cuda")
    ws = msa.workspace(msa.msa_gather_device_workspace_size(B, k, cap))
    msa.msa_gather_device(ctx128, host, row_bytes, N, coff_dev, torch.from_numpy(ids).cuda(), dst, cap, mo, ws)
    # the host-side gather of the same ids gives the same bytes and offsets
    dst2 = torch.zeros_like(dst)
    mo_h = torch.zeros(B + 1, dtype=torch.int64, pin_memory=True)
    side = torch.cuda.Stream()
    msa.msa_gather(host, row_bytes, N, coff, ids, k, dst2, cap, mo_h, side=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    mo_np = mo.cpu().numpy()
    assert np.array_equal(mo_np, mo_h.numpy())
    got = W.host_bits(dst)
    assert np.array_equal(got, W.host_bits(dst2))
    for b in range(B):
        ref, m = oracle.gather_rows(bank, coff, ids[b])
        assert mo_np[b + 1] - mo_np[b] == m
        assert np.array_equal(got[mo_np[b]:mo_np[b + 1]], ref)


def _random_gather_cases(n, seed):
    """Seeded layouts: rows of 256 B to 8 KiB (K and V of 1-8 heads, d 64 or
    128, bf16 or fp32 elements; the copy is byte-level), 1-200 documents of
    1-20 chunk rows, 1-4 queries, k up to 64, ids in random order with a run
    of consecutive ids in some rows."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        row_elems = 2 * int(rng.choice([1, 2, 4, 8])) * int(rng.choice([64, 128])) * int(rng.choice([1, 2]))
        n_docs = int(rng.integers(1, 201))
        B = int(rng.integers(1, 5))
        k = int(rng.integers(1, min(n_docs, 64) + 1))
        cases.append((row_elems, n_docs, int(rng.integers(1, 21)), B, k, 900 + i))
    return cases


@pytest.mark.parametrize("row_elems,n_docs,maxc,B,k,seed", _random_gather_cases(10, 63))
def test_gather_random_layouts(torch_mod, msa, ctx128, row_elems, n_docs, maxc, B, k, seed):
    torch = torch_mod
    rng = np.random.default_rng(seed)
    coff = msa_synth.prefix_offsets(rng.integers(1, maxc + 1, size=n_docs))
    N = int(coff[-1])
    bank = msa_synth.counter_bf16(seed, 8, 0, N * row_elems).reshape(N, row_elems)
    host = torch.empty((N, row_elems), dtype=torch.bfloat16, pin_memory=True)
    host.copy_(W.dev_bf16(bank, "cpu"))
    ids = np.stack([rng.permutation(n_docs)[:k] for _ in range(B)]).astype(np.int32)
    for b in range(0, B, 2):                       # a run of consecutive documents
        if k >= 3 and n_docs >= k:
            start = int(rng.integers(0, n_docs - k + 1))
            ids[b] = np.arange(start, start + k, dtype=np.int32)[rng.permutation(k)]
    cap = int(sum(np.diff(coff)[ids[b]].sum() for b in range(B)))
    row_bytes = row_elems * 2
    dst = torch.zeros((cap, row_elems), dtype=torch.bfloat16, device="cuda")
    mo = torch.zeros(B + 1, dtype=torch.int64, device="cuda")
    ws = msa.workspace(msa.msa_gather_device_workspace_size(B, k, cap))
    msa.msa_gather_device(ctx128, host, row_bytes, N, torch.from_numpy(coff).cuda(),
                          torch.from_numpy(ids).cuda(), dst, cap, mo, ws)
    dst2 = torch.zeros_like(dst)
    mo_h = torch.zeros(B + 1, dtype=torch.int64, pin_memory=True)
    side = torch.cuda.Stream()
    msa.msa_gather(host, row_bytes, N, coff, ids, k, dst2, cap, mo_h, side=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    mo_np = mo.cpu().numpy()
    assert np.array_equal(mo_np, mo_h.numpy())
    got, got2 = W.host_bits(dst), W.host_bits(dst2)
    for b in range(B):
        ref, m = oracle.gather_rows(bank, coff, ids[b])
        assert mo_np[b + 1] - mo_np[b] == m
        assert np.array_equal(got[mo_np[b]:mo_np[b + 1]], ref)
        assert np.array_equal(got2[mo_np[b]:mo_np[b + 1]], ref)
    assert mo_np[B] == cap


@pytest.mark.parametrize("B", [64, 65])
def test_gather_device_both_plans(torch_mod, msa, ctx128, B):
    """64 queries take the plan with one workgroup per query, 65 the plan
    with one workgroup for all: the same rows and offsets as the oracle's
    indexing either way, with an invalid id and a capacity that cuts the
    last query short."""
    torch = torch_mod
    rng = np.random.default_rng(300 + B)
    n_docs, k, row_elems = 300, 12, 64
    coff = msa_synth.prefix_offsets(rng.integers(1, 9, size=n_docs))
    N = int(coff[-1])
    bank = msa_synth.counter_bf16(300 + B, 3, 0, N * row_elems).reshape(N, row_elems)
    host = torch.empty((N, row_elems), dtype=torch.bfloat16, pin_memory=True)
    host.copy_(W.dev_bf16(bank, "cpu"))
    ids = np.stack([rng.permutation(n_docs)[:k] for _ in range(B)]).astype(np.int32)
    ids[3, 5] = -1                                   # an invalid id copies nothing
    valid = [ids[b][ids[b] >= 0] for b in range(B)]
    full = int(sum(np.diff(coff)[v].sum() for v in valid))
    cap = full - 3                                   # the last query's rows cut short
    dst = torch.zeros((cap, row_elems), dtype=torch.bfloat16, device="cuda")
    mo = torch.zeros(B + 1, dtype=torch.int64, device="cuda")
    ws = msa.workspace(msa.msa_gather_device_workspace_size(B, k, cap))
    msa.msa_gather_device(ctx128, host, row_elems * 2, N, torch.from_numpy(coff).cuda(),
                          torch.from_numpy(ids).cuda(), dst, cap, mo, ws)
    torch.cuda.synchronize()
    mo_np = mo.cpu().numpy()
    got = W.host_bits(dst)
    start = 0
    for b in range(B):
        ref, m = oracle.gather_rows(bank, coff, valid[b])
        end = min(start + m, cap)
        assert mo_np[b] == min(start, cap) and mo_np[b + 1] == end, b
        assert np.array_equal(got[start:end], ref[:end - start]), b
        start += m
    assert mo_np[B] == cap


def test_gather_device_skips_invalid_ids_and_clamps_to_capacity(torch_mod, msa, ctx128):
    torch = torch_mod
    coff = np.array([0, 3, 5, 9, 10], dtype=np.int64)
    bank = msa_synth.counter_bf16(5, 7, 0, 10 * 64).reshape(10, 64)
    host = torch.empty((10, 64), dtype=torch.bfloat16, pin_memory=True)
    host.copy_(W.dev_bf16(bank, "cpu"))
    ids = torch.tensor([[2, -5, 0], [99, 3, 1]], dtype=torch.int32, device="cuda")
    cap = 8
    dst = torch.zeros((cap, 64), dtype=torch.bfloat16, device="cuda")
    mo = torch.zeros(3, dtype=torch.int64, device="cuda")
    ws = msa.workspace(msa.msa_gather_device_workspace_size(2, 3, cap))
    msa.msa_gather_device(ctx128, host, 128, 10, torch.from_numpy(coff).cuda(), ids, dst, cap, mo, ws)
    torch.cuda.synchronize()
    # query 0: docs 0 (3 rows) and 2 (4 rows) -> 7 rows; query 1: docs 1, 3 -> clamped to 1 row
    assert mo.cpu().tolist() == [0, 7, 8]
    got = W.host_bits(dst)
    assert np.array_equal(got[:3], bank[0:3]) and np.array_equal(got[3:7], bank[5:9])
    assert np.array_equal(got[7:8], bank[3:4])


def test_gather_device_one_query_skips_invalid_ids_and_clamps_to_capacity(torch_mod, msa, ctx128):
    """The single-query gather (one launch) follows the same rules as the
    batched one: ids outside [0, n_docs) are skipped, the selected documents
    are laid out in ascending id order, and rows past cap_rows are dropped."""
    torch = torch_mod
    coff = np.array([0, 3, 5, 9, 10], dtype=np.int64)
    bank = msa_synth.counter_bf16(5, 9, 0, 10 * 64).reshape(10, 64)
    host = torch.empty((10, 64), dtype=torch.bfloat16, pin_memory=True)
    host.copy_(W.dev_bf16(bank, "cpu"))
    for ids_row, cap, want_rows, want in [
        ([2, -5, 0, 99], 8, 7, [bank[0:3], bank[5:9]]),          # invalid ids skipped
        ([3, 1, 2], 5, 5, [bank[3:5], bank[5:8]]),                # doc 2's last row and doc 3 past the cap
    ]:
        ids = torch.tensor([ids_row], dtype=torch.int32, device="cuda")
        dst = torch.zeros((cap, 64), dtype=torch.bfloat16, device="cuda")
        mo = torch.zeros(2, dtype=torch.int64, device="cuda")
        ws = msa.workspace(msa.msa_gather_device_workspace_size(1, len(ids_row), cap))
        msa.msa_gather_device(ctx128, host, 128, 10, torch.from_numpy(coff).cuda(), ids, dst, cap, mo, ws)
        torch.cuda.synchronize()
        assert mo.cpu().tolist() == [0, want_rows]
        assert np.array_equal(W.host_bits(dst)[:want_rows], np.concatenate(want))


def test_gather_device_one_query_past_the_single_launch_size(torch_mod, msa, ctx128):
    """One query whose selected documents fill more than 8,192 destination
    rows takes the plan + copy kernels instead of the single launch; the bytes
    and offsets must match the oracle's indexing either way."""
    torch = torch_mod
    rng = np.random.default_rng(71)
    n_docs, k, row_elems = 200, 60, 64
    coff = msa_synth.prefix_offsets(rng.integers(120, 200, size=n_docs))
    N = int(coff[-1])
    bank = msa_synth.counter_bf16(71, 3, 0, N * row_elems).reshape(N, row_elems)
    host = torch.empty((N, row_elems), dtype=torch.bfloat16, pin_memory=True)
    host.copy_(W.dev_bf16(bank, "cpu"))
    ids = rng.permutation(n_docs)[:k].astype(np.int32)[None]
    cap = int(np.diff(coff)[ids[0]].sum())
    assert cap > 8192
    dst = torch.zeros((cap, row_elems), dtype=torch.bfloat16, device="cuda")
    mo = torch.zeros(2, dtype=torch.int64, device="cuda")
    ws = msa.workspace(msa.msa_gather_device_workspace_size(1, k, cap))
    msa.msa_gather_device(ctx128, host, row_elems * 2, N, torch.from_numpy(coff).cuda(),
                          torch.from_numpy(ids).cuda(), dst, cap, mo, ws)
    torch.cuda.synchronize()
    ref, m = oracle.gather_rows(bank, coff, ids[0])
    assert mo.cpu().tolist() == [0, m] and m == cap
    assert np.array_equal(W.host_bits(dst), ref)
