"""Backward of the document score on the GPU vs the oracle, through the C ABI.

Tolerances (stated where used):
  arg max   (chunk, token) of every document bit-exact, on inputs whose best
            and second-best (chunk, token) scores differ by more than 1e-4
            (checked here with the oracle); the GPU compares fp32 scores
            whose error is below 1e-5 (the fp32 group fold of the forward).
  grads     1e-4 of max |ref| per tensor: fp32 sums of unit vectors scaled by
            the document gradients, from inputs the oracle widens exactly.
"""

import numpy as np
import pytest

import msa_synth
import oracle
from tests import workloads as W

pytestmark = pytest.mark.gpu

MARGIN = 1e-4
GRAD_TOL = 1e-4


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
def ctxs(msa):
    c = {128: msa.msa_ctx_create(0, 128, 1e6, 16384), 64: msa.msa_ctx_create(0, 64, 1e4, 4096)}
    yield c
    for v in c.values():
        v.close()


def _margins_ok(Qr, Kr, off):
    s = oracle.pair_scores(Qr, Kr)
    for doc in range(len(off) - 1):
        blk = s[:, off[doc]:off[doc + 1], :].reshape(s.shape[0], -1)
        if blk.shape[1] > 1:
            top2 = np.sort(blk, axis=1)[:, -2:]
            if np.min(top2[:, 1] - top2[:, 0]) <= MARGIN:
                return False
    return True


def _rel(got, ref):
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


CASES = [
    # dtype, d, Hq, Hkv, B, Tq, chunks per document, zero-gradient documents
    ("f32", 64, 4, 2, 1, 32, [16] * 64, [3, 40]),                 # tiny fp32 shape (64 docs x 16 chunks)
    ("bf16", 128, 32, 8, 2, 16, [2, 16, 5, 9, 1, 12] * 8, [0]),   # Qwen3-4B-shaped heads, ragged documents
    ("bf16", 128, 32, 8, 4, 1, [1] * 300, []),                    # chunk-level selection, one decode token
    ("bf16", 128, 64, 16, 1, 8, [4, 7, 3] * 10, [5]),             # Hkv 16: rows of 2,048 elements
    ("f32", 64, 2, 1, 3, 5, [3, 1, 8] * 7, [1, 2]),               # Hkv 1, d 64: rows of 64 elements
    ("bf16", 128, 32, 8, 1, 4, [40, 3], []),                      # a document staged in several blocks
]


def _random_cases(n, seed):
    """Seeded shapes: either dtype and head dim, KV heads 1-16 with group
    sizes 1-8, 1-3 queries of 1-16 tokens, 1-60 documents of 1-20 chunks, and
    a few documents whose score gradient is zero."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = ("bf16", "f32")[i % 2]
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4, 8, 16]))
        G = int(rng.choice([1, 2, 4, 8]))
        n_docs = int(rng.integers(1, 61))
        lens = [int(x) for x in rng.integers(1, 21, size=n_docs)]
        zero = sorted(int(x) for x in rng.choice(n_docs, size=int(rng.integers(0, min(3, n_docs) + 1)),
                                                   replace=False))
        cases.append((dtype, d, G * Hkv, Hkv, int(rng.integers(1, 4)), int(rng.integers(1, 17)), lens, zero))
    return cases


@pytest.mark.parametrize("dtype,d,Hq,Hkv,B,Tq,lens,zero_docs", CASES + _random_cases(8, 31))
def test_route_bwd_parity(torch_mod, msa, ctxs, dtype, d, Hq, Hkv, B, Tq, lens, zero_docs):
    torch = torch_mod
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    N, n_docs = int(off[-1]), len(lens)
    for seed in range(101, 111):                 # the first seed whose arg maxes have a margin
        Qr = W.draw(seed, 1, (B, Tq, Hq, d), dtype)
        Kr = W.draw(seed, 2, (N, Hkv, d), dtype)
        if _margins_ok(W.widen(Qr, dtype), W.widen(Kr, dtype), off):
            break
    else:
        pytest.fail("no seed with arg-max margins")
    print(f"\nroute bwd case {dtype} d={d} Hq={Hq} Hkv={Hkv} B={B} Tq={Tq} docs={n_docs} seed={seed}", flush=True)
    dscore = msa_synth.normal_f32(seed, 3, (B, n_docs)).astype(np.float32)
    dscore[:, zero_docs] = 0.0
    dQr = torch.full((B, Tq, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    dKr = torch.full((N, Hkv, d), float("nan"), dtype=torch.float32, device="cuda")
    arg = torch.full((B, n_docs, 2), -7, dtype=torch.int32, device="cuda")
    ws = msa.workspace(msa.msa_route_bwd_workspace_size(B, Tq, Hq, Hkv, N, n_docs))
    msa.msa_route_bwd(ctxs[d], W.dev(Qr, dtype), W.dev(Kr, dtype), torch.from_numpy(off).cuda(),
                      torch.from_numpy(dscore).cuda(), dQr, dKr, ws, out_arg=arg)
    torch.cuda.synchronize()
    q64, k64 = W.widen(Qr, dtype), W.widen(Kr, dtype)
    _, ac, at = oracle.doc_score_argmax(q64, k64, off)
    got_arg = arg.cpu().numpy()
    live = dscore != 0
    assert np.array_equal(got_arg[..., 0][live], ac[live])
    assert np.array_equal(got_arg[..., 1][live], at[live])
    assert np.all(got_arg[~live] == -1)
    rq, rk = oracle.route_score_bwd(q64, k64, off, dscore.astype(np.float64))
    gq, gk = dQr.cpu().numpy(), dKr.cpu().numpy()
    print(f"dQr rel {_rel(gq, rq):.2e}  dKr rel {_rel(gk, rk):.2e}", flush=True)
    assert np.all(np.isfinite(gq)) and np.all(np.isfinite(gk))
    assert _rel(gq, rq) <= GRAD_TOL
    assert _rel(gk, rk) <= GRAD_TOL


def test_route_bwd_zero_vectors(torch_mod, msa, ctxs):
    """A zero routing-key row and a zero query head: the clamped norm is a
    constant there (the oracle's reading), so the gradient is k^/eps or
    q^/eps-scaled and finite."""
    torch = torch_mod
    B, Tq, Hq, Hkv, d = 1, 2, 4, 2, 64
    off = np.array([0, 3, 5], dtype=np.int64)
    Qr = msa_synth.normal_f32(7, 1, (B, Tq, Hq, d)).astype(np.float32)
    Kr = msa_synth.normal_f32(7, 2, (5, Hkv, d)).astype(np.float32)
    Qr[0, 1, 3] = 0.0
    Kr[4, 1] = 0.0
    for k in range(5):                          # chunk k aligned with token k % 2 to give margins
        Kr[k] += 3.0 * Qr[0, k % 2].reshape(Hkv, Hq // Hkv, d).sum(axis=1) * (k + 1) / 5
    Kr[4, 1] = 0.0
    assert _margins_ok(Qr.astype(np.float64), Kr.astype(np.float64), off)
    dscore = np.array([[0.7, -1.3]], dtype=np.float32)
    dQr = torch.empty((B, Tq, Hq, d), dtype=torch.float32, device="cuda")
    dKr = torch.empty((5, Hkv, d), dtype=torch.float32, device="cuda")
    ws = msa.workspace(msa.msa_route_bwd_workspace_size(B, Tq, Hq, Hkv, 5, 2))
    msa.msa_route_bwd(ctxs[64], W.dev_f32(Qr), W.dev_f32(Kr), torch.from_numpy(off).cuda(),
                      torch.from_numpy(dscore).cuda(), dQr, dKr, ws)
    torch.cuda.synchronize()
    rq, rk = oracle.route_score_bwd(Qr.astype(np.float64), Kr.astype(np.float64), off, dscore.astype(np.float64))
    gq, gk = dQr.cpu().numpy(), dKr.cpu().numpy()
    assert np.all(np.isfinite(gq)) and np.all(np.isfinite(gk))
    assert _rel(gq, rq) <= GRAD_TOL and _rel(gk, rk) <= GRAD_TOL


def test_route_bwd_is_deterministic(torch_mod, msa, ctxs):
    torch = torch_mod
    off = np.concatenate([[0], np.cumsum([3, 9, 1, 4] * 20)]).astype(np.int64)
    N = int(off[-1])
    Qr = W.dev_bf16(msa_synth.normal_bf16(13, 1, (3, 16, 32, 128)))
    Kr = W.dev_bf16(msa_synth.normal_bf16(13, 2, (N, 8, 128)))
    dscore = torch.from_numpy(msa_synth.normal_f32(13, 3, (3, 80)).astype(np.float32)).cuda()
    ws = msa.workspace(msa.msa_route_bwd_workspace_size(3, 16, 32, 8, N, 80))
    outs = []
    for _ in range(2):
        dQr = torch.empty((3, 16, 32, 128), dtype=torch.float32, device="cuda")
        dKr = torch.empty((N, 8, 128), dtype=torch.float32, device="cuda")
        msa.msa_route_bwd(ctxs[128], Qr, Kr, torch.from_numpy(off).cuda(), dscore, dQr, dKr, ws)
        outs.append((dQr.cpu().numpy(), dKr.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_route_bwd_full_size_routebwd1m(torch_mod, msa, ctxs):
    """The shape and inputs the bench's routing training pass times: a
    256-token query over the 1M-token memory of 2,000 documents (lengths
    uniform in [128, 1024], chunk 64, 19,254 chunk rows), dense dscore.
    Documents whose best two (chunk, token) scores are within 1e-4 (by the
    oracle) get dscore = 0, so every remaining arg max is unique."""
    from msa_synth import device as device_fill
    torch = torch_mod
    seed, T, Hq, Hkv, d = 0, 256, 32, 8, 128
    lens = msa_synth.uniform_lengths(seed, 2000, 128, 1024)
    coff = msa_synth.prefix_offsets([(int(x) + 63) // 64 for x in lens])
    n_docs, N = len(lens), int(coff[-1])
    Qr_d = torch.empty((1, T, Hq, d), dtype=torch.bfloat16, device="cuda")
    Kr_d = torch.empty((N, Hkv, d), dtype=torch.bfloat16, device="cuda")
    device_fill.fill_counter_bf16(Qr_d, seed, 730, 0)
    device_fill.fill_counter_bf16(Kr_d, seed, 731, 0)
    q64 = W.widen(W.counter_bf16_threads(seed, 730, 0, T * Hq * d).reshape(1, T, Hq, d), "bf16")
    k64 = W.widen(W.counter_bf16_threads(seed, 731, 0, N * Hkv * d).reshape(N, Hkv, d), "bf16")
    dscore = msa_synth.normal_f32(seed, 732, (1, n_docs)).astype(np.float32)
    # margins from the oracle's score of every (chunk, token) pair
    s = oracle.pair_scores(q64, k64)[0]                                                       # [N, T]
    for doc in range(n_docs):
        blk = np.sort(s[coff[doc]:coff[doc + 1]].ravel())
        if blk[-1] - blk[-2] <= 1e-4:
            dscore[0, doc] = 0.0
    live = dscore[0] != 0
    print(f"\nfull-size route bwd: {int(live.sum())} of {n_docs} documents carry a gradient", flush=True)
    assert live.sum() > 0.9 * n_docs
    dQr = torch.empty((1, T, Hq, d), dtype=torch.float32, device="cuda")
    dKr = torch.empty((N, Hkv, d), dtype=torch.float32, device="cuda")
    arg = torch.empty((1, n_docs, 2), dtype=torch.int32, device="cuda")
    ws = msa.workspace(msa.msa_route_bwd_workspace_size(1, T, Hq, Hkv, N, n_docs))
    msa.msa_route_bwd(ctxs[128], Qr_d, Kr_d, torch.from_numpy(coff).cuda(), torch.from_numpy(dscore).cuda(),
                      dQr, dKr, ws, out_arg=arg)
    torch.cuda.synchronize()
    _, ac, at = oracle.doc_score_argmax(q64, k64, coff)
    got = arg.cpu().numpy()
    assert np.array_equal(got[0, live, 0], ac[0, live]) and np.array_equal(got[0, live, 1], at[0, live])
    rq, rk = oracle.route_score_bwd(q64, k64, coff, dscore.astype(np.float64))
    gq, gk = dQr.cpu().numpy(), dKr.cpu().numpy()
    print(f"dQr rel {_rel(gq, rq):.2e}  dKr rel {_rel(gk, rk):.2e}", flush=True)
    assert _rel(gq, rq) <= GRAD_TOL and _rel(gk, rk) <= GRAD_TOL


def test_route_bwd_validation_errors(torch_mod, msa, ctxs):
    torch = torch_mod
    Qr = torch.zeros((1, 2, 32, 128), dtype=torch.bfloat16, device="cuda")
    Kr = torch.zeros((6, 8, 128), dtype=torch.bfloat16, device="cuda")
    off = torch.tensor([0, 3, 6], dtype=torch.int64, device="cuda")
    ds = torch.ones((1, 2), dtype=torch.float32, device="cuda")
    dQ = torch.empty((1, 2, 32, 128), dtype=torch.float32, device="cuda")
    dK = torch.empty((6, 8, 128), dtype=torch.float32, device="cuda")
    ws = msa.workspace(msa.msa_route_bwd_workspace_size(1, 2, 32, 8, 6, 2))
    with pytest.raises(msa.MsaError) as e:                       # Hq % Hkv
        msa.msa_route_bwd(ctxs[128], Qr[:, :, :30].contiguous(), Kr, off, ds, dQ[:, :, :30].contiguous(), dK, ws)
    assert e.value.status == msa.MSA_ERR_INVALID_ARG
    with pytest.raises(msa.MsaError) as e:                       # workspace too small
        msa.msa_route_bwd(ctxs[128], Qr, Kr, off, ds, dQ, dK, msa.workspace(256))
    assert e.value.status == msa.MSA_ERR_WORKSPACE
    Kr12 = torch.zeros((6, 12, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(msa.MsaError) as e:                       # Hkv * d not a power of two
        msa.msa_route_bwd(ctxs[128], Qr[:, :, :24].contiguous(), Kr12, off, ds, dQ[:, :, :24].contiguous(),
                          torch.empty((6, 12, 128), dtype=torch.float32, device="cuda"), ws)
    assert e.value.status == msa.MSA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
