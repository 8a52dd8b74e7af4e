"""Backward of the sparse attention on the GPU vs the oracle, through the C ABI.

Tolerances (stated where used):
  lse      2e-2 absolute in bf16, 1e-3 in fp32: the logits the forward
           exponentiates carry the bf16 rounding of the rotated, scaled
           query and of the rotated local keys (relative 2^-9 per element), a
           random-sign error of about sqrt(d) * 2^-9 * scale |q_c k_c| ~ 3e-3
           on unit-variance inputs; the log-sum-exp inherits at most the
           largest logit error.
  grads    2e-2 of max |ref| per gradient tensor (the bf16 attention bar):
           the GPU recomputes P from bf16 operands and the bf16 forward output
           (D = dO . O), contracts bf16 P, dS, dO, Q and K with fp32
           accumulation and stores bf16, each a relative 2^-9 rounding.
"""

import numpy as np
import pytest

import msa_synth
import oracle
from tests import workloads as W

pytestmark = pytest.mark.gpu

LSE_TOL = {"bf16": 2e-2, "f32": 1e-3}
GRAD_TOL = 2e-2


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


def _inputs(seed, dtype, d, Hq, Hkv, B, Tq, L, rows):
    mem_off = msa_synth.prefix_offsets(rows)
    M = int(mem_off[-1])
    return dict(mem_off=mem_off, M=M,
                Q=W.draw(seed, 1, (B, Tq, Hq, d), dtype),
                KV=W.draw(seed, 2, (max(M, 1), 2, Hkv, d), dtype),
                Kl=W.draw(seed, 3, (B, L, Hkv, d), dtype),
                Vl=W.draw(seed, 4, (B, L, Hkv, d), dtype),
                dO=W.draw(seed, 5, (B, Tq, Hq, d), dtype))


def _forward_lse(torch, msa, ctx, x, dtype, rows, qoff):
    B, Tq, Hq, d = x["Q"].shape
    L, Hkv = x["Kl"].shape[1:3]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = {k: W.dev(x[k], dtype) for k in ("Q", "KV", "Kl", "Vl")}
    O = torch.full((B, Tq, Hq, d), float("nan"), dtype=tdt, device="cuda")
    lse = torch.full((B, Tq, Hq), float("nan"), dtype=torch.float32, device="cuda")
    mo = torch.from_numpy(x["mem_off"]).cuda()
    ws = msa.workspace(msa.msa_sparse_attn_workspace_size(1 if dtype == "bf16" else 0, B, Tq, Hq, Hkv,
                                                          max(rows), L))
    msa.msa_sparse_attn_lse(ctx, dev["Q"], dev["KV"], mo, max(rows), dev["Kl"], dev["Vl"], qoff,
                            W.scale_of(d), O, lse, ws)
    return dev, mo, O, lse


LSE_CASES = [
    # dtype, d, Hq, Hkv, B, Tq, L, rows per query, q_offset
    ("bf16", 128, 32, 8, 1, 256, 256, [152], 16),     # matrix-core prefill path
    ("bf16", 128, 32, 8, 2, 200, 500, [0, 300], 16),  # matrix cores, partial tile
    ("bf16", 128, 32, 8, 3, 1, 700, [30, 0, 300], 16),  # decode path
    ("f32", 64, 4, 2, 1, 32, 32, [64], 4),            # generic split path
    ("bf16", 128, 16, 1, 1, 7, 19, [260], 33),        # generic split path, G = 16
]


@pytest.mark.parametrize("dtype,d,Hq,Hkv,B,Tq,L,rows,qoff", LSE_CASES)
def test_sparse_attn_lse_parity(torch_mod, msa, ctx64, ctx128, dtype, d, Hq, Hkv, B, Tq, L, rows, qoff):
    torch = torch_mod
    ctx = ctx128 if d == 128 else ctx64
    x = _inputs(91, dtype, d, Hq, Hkv, B, Tq, L, rows)
    _, _, O, lse = _forward_lse(torch, msa, ctx, x, dtype, rows, qoff)
    torch.cuda.synchronize()
    kv = W.widen(x["KV"], dtype)
    args = (W.widen(x["Q"], dtype), kv[:, 0], kv[:, 1], x["mem_off"], W.widen(x["Kl"], dtype),
            W.widen(x["Vl"], dtype), qoff, W.scale_of(d), ctx.rope_theta)
    ref_lse = oracle.sparse_attn_lse(*args)
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) <= LSE_TOL[dtype]
    ref_o = oracle.sparse_attn(*args)            # the output is unchanged by saving lse
    assert np.max(np.abs(W.widen(W.host_bits(O), dtype) - ref_o)) <= (2e-2 if dtype == "bf16" else 1e-3)


BWD_CASES = [
    # Hq, Hkv, B, Tq, L, rows per query, q_offset
    (32, 8, 1, 64, 600, [250], 32),        # G = 4, several key tiles, causal edge
    (32, 8, 2, 200, 500, [0, 300], 16),    # partial query tile, one query without memory
    (8, 8, 1, 130, 130, [70], 8),          # G = 1, Tq = L, ragged tiles
    (16, 1, 1, 96, 1000, [64], 16),        # G = 16: four workgroups per query tile
    (64, 8, 2, 1, 700, [90, 200], 16),     # one query token (decode shape), G = 8
    (4, 2, 1, 33, 40, [5], 4),             # G = 2, one token past a tile
    (32, 8, 2, 1, 1, [0, 5], 16),          # one local key; one query sees only it
    (32, 8, 1, 300, 300, [1], 16),         # Tq = L, one memory row
]


def _random_bwd_cases(n, seed):
    """Seeded shapes: G cycling through 1, 2, 4 and 8, 1-2 queries of 1-150
    tokens, ragged memory rows (some queries without any), local lengths up to
    400 and offsets k, so query and key tiles end at every alignment."""
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        G = (1, 2, 4, 8)[k % 4]
        Hkv = int(rng.choice([1, 2, 4]))
        B = int(rng.integers(1, 3))
        Tq = int(rng.integers(1, 151))
        L = int(rng.integers(Tq, 401))
        rows = [int(r) if rng.random() > 0.25 else 0 for r in rng.integers(0, 300, size=B)]
        cases.append((G * Hkv, Hkv, B, Tq, L, rows, int(rng.integers(0, 41))))
    return cases


def _rel(got, ref):
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


@pytest.mark.parametrize("Hq,Hkv,B,Tq,L,rows,qoff", BWD_CASES + _random_bwd_cases(8, 77))
def test_sparse_attn_bwd_parity(torch_mod, msa, ctx128, Hq, Hkv, B, Tq, L, rows, qoff):
    torch = torch_mod
    d = 128
    print(f"\nbwd case Hq={Hq} Hkv={Hkv} B={B} Tq={Tq} L={L} rows={rows}", flush=True)
    x = _inputs(93, "bf16", d, Hq, Hkv, B, Tq, L, rows)
    dev, mo, O, lse = _forward_lse(torch, msa, ctx128, x, "bf16", rows, qoff)
    dO = W.dev_bf16(x["dO"])
    nan = lambda t: torch.full_like(t, float("nan"))
    dQ, dKV, dKl, dVl = nan(dev["Q"]), nan(dev["KV"]), nan(dev["Kl"]), nan(dev["Vl"])
    ws = msa.workspace(msa.msa_sparse_attn_bwd_workspace_size(1, B, Tq, Hq, Hkv, max(rows), L))
    msa.msa_sparse_attn_bwd(ctx128, dev["Q"], dev["KV"], mo, max(rows), dev["Kl"], dev["Vl"], qoff,
                            W.scale_of(d), O, dO, lse, dQ, dKV, dKl, dVl, ws)
    torch.cuda.synchronize()
    kv = W.widen(x["KV"], "bf16")
    ref = oracle.sparse_attn_bwd(W.widen(x["Q"], "bf16"), kv[:, 0], kv[:, 1], x["mem_off"],
                                 W.widen(x["Kl"], "bf16"), W.widen(x["Vl"], "bf16"), qoff, W.scale_of(d),
                                 ctx128.rope_theta, W.widen(x["dO"], "bf16"))
    dkv = W.widen(W.host_bits(dKV), "bf16")
    M = x["M"]
    got = [W.widen(W.host_bits(dQ), "bf16"), dkv[:M, 0], dkv[:M, 1],
           W.widen(W.host_bits(dKl), "bf16"), W.widen(W.host_bits(dVl), "bf16")]
    want = [ref[0], ref[1][:M], ref[2][:M], ref[3], ref[4]]
    for name, g, r in zip(["dQ", "dK_mem", "dV_mem", "dK_local", "dV_local"], got, want):
        if r.size == 0:
            continue
        assert np.all(np.isfinite(g)), name
        print(f"{name}: rel max err {_rel(g, r):.3e}", flush=True)
        assert _rel(g, r) <= GRAD_TOL, (name, _rel(g, r))


def test_sparse_attn_bwd_leaves_other_memory_rows_alone(torch_mod, msa, ctx128):
    # query 0 reads rows 10..29 and query 1 rows 30..69 of an 80-row buffer:
    # rows 0..9 and 70..79 belong to nobody and must keep their contents
    torch = torch_mod
    x = _inputs(95, "bf16", 128, 32, 8, 2, 40, 80, [20, 40])
    mem_off = np.array([10, 30, 70], dtype=np.int64)
    KV = W.draw(95, 6, (80, 2, 8, 128), "bf16")
    Q, Kl, Vl, KVd = W.dev_bf16(x["Q"]), W.dev_bf16(x["Kl"]), W.dev_bf16(x["Vl"]), W.dev_bf16(KV)
    mo = torch.from_numpy(mem_off).cuda()
    O = torch.empty_like(Q)
    lse = torch.empty((2, 40, 32), dtype=torch.float32, device="cuda")
    ws = msa.workspace(msa.msa_sparse_attn_workspace_size(1, 2, 40, 32, 8, 40, 80))
    msa.msa_sparse_attn_lse(ctx128, Q, KVd, mo, 40, Kl, Vl, 16, W.scale_of(128), O, lse, ws)
    dQ, dKl, dVl = torch.empty_like(Q), torch.empty_like(Kl), torch.empty_like(Vl)
    dKV = torch.full_like(KVd, 1.0)
    sentinel = 0x3F80                                     # bf16 1.0
    wsb = msa.workspace(msa.msa_sparse_attn_bwd_workspace_size(1, 2, 40, 32, 8, 40, 80))
    msa.msa_sparse_attn_bwd(ctx128, Q, KVd, mo, 40, Kl, Vl, 16, W.scale_of(128), O, W.dev_bf16(x["dO"]), lse,
                            dQ, dKV, dKl, dVl, wsb)
    torch.cuda.synchronize()
    bits = W.host_bits(dKV)
    assert np.all(bits[:10] == sentinel) and np.all(bits[70:] == sentinel)
    kv = W.widen(KV, "bf16")
    ref = oracle.sparse_attn_bwd(W.widen(x["Q"], "bf16"), kv[:, 0], kv[:, 1], mem_off,
                                 W.widen(x["Kl"], "bf16"), W.widen(x["Vl"], "bf16"), 16, W.scale_of(128),
                                 ctx128.rope_theta, W.widen(x["dO"], "bf16"))
    got = W.widen(bits, "bf16")
    assert _rel(got[10:70, 0], ref[1][10:70]) <= GRAD_TOL
    assert _rel(got[10:70, 1], ref[2][10:70]) <= GRAD_TOL


def test_sparse_attn_bwd_is_deterministic(torch_mod, msa, ctx128):
    torch = torch_mod
    x = _inputs(97, "bf16", 128, 32, 8, 1, 96, 300, [100])
    dev, mo, O, lse = _forward_lse(torch, msa, ctx128, x, "bf16", [100], 16)
    ws = msa.workspace(msa.msa_sparse_attn_bwd_workspace_size(1, 1, 96, 32, 8, 100, 300))
    outs = []
    for _ in range(2):
        g = [torch.empty_like(dev["Q"]), torch.empty_like(dev["KV"]), torch.empty_like(dev["Kl"]),
             torch.empty_like(dev["Vl"])]
        msa.msa_sparse_attn_bwd(ctx128, dev["Q"], dev["KV"], mo, 100, dev["Kl"], dev["Vl"], 16,
                                W.scale_of(128), O, W.dev_bf16(x["dO"]), lse, *g, ws)
        outs.append([W.host_bits(t) for t in g])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_sparse_attn_bwd_rejects_unsupported(torch_mod, msa, ctx64):
    torch = torch_mod
    x = _inputs(99, "bf16", 64, 4, 2, 1, 4, 8, [3])
    dev = {k: W.dev_bf16(x[k]) for k in ("Q", "KV", "Kl", "Vl", "dO")}
    lse = torch.zeros((1, 4, 4), dtype=torch.float32, device="cuda")
    mo = torch.tensor([0, 3], dtype=torch.int64, device="cuda")
    ws = msa.workspace(1 << 20)
    with pytest.raises(msa.MsaError) as e:                       # head dim 64
        msa.msa_sparse_attn_bwd(ctx64, dev["Q"], dev["KV"], mo, 3, dev["Kl"], dev["Vl"], 4, 0.125,
                                dev["Q"], dev["dO"], lse, torch.empty_like(dev["Q"]),
                                torch.empty_like(dev["KV"]), torch.empty_like(dev["Kl"]),
                                torch.empty_like(dev["Vl"]), ws)
    assert e.value.status == msa.MSA_ERR_UNSUPPORTED


def test_sparse_attn_bwd_full_size_sampled(torch_mod, msa, ctx128):
    """The training-pass shape and launch the bench times: 8,192 tokens over
    [242 memory rows ; 8,192 local keys], Hq 32, Hkv 8, inputs from the same
    counter streams.  Sampled outputs of one KV group against the oracle:
    dQ of 40 tokens (first, ragged middle, last) for the group's four heads,
    dK and dV of 48 keys (memory rows, the memory/local boundary, the last
    local keys)."""
    from msa_synth import device as device_fill
    torch = torch_mod
    seed, T, M, qoff, Hq, Hkv, d = 0, 8192, 242, 32, 32, 8, 128
    shapes = {"Q": (1, T, Hq, d), "KV": (M, 2, Hkv, d), "Kl": (1, T, Hkv, d), "Vl": (1, T, Hkv, d),
              "dO": (1, T, Hq, d)}
    streams = {"Q": 720, "KV": 721, "Kl": 722, "Vl": 723, "dO": 724}
    dev = {}
    for k, shp in shapes.items():
        dev[k] = torch.empty(shp, dtype=torch.bfloat16, device="cuda")
        device_fill.fill_counter_bf16(dev[k], seed, streams[k], 0)
    mo = torch.tensor([0, M], dtype=torch.int64, device="cuda")
    O = torch.empty_like(dev["Q"])
    lse = torch.empty((1, T, Hq), dtype=torch.float32, device="cuda")
    ws = msa.workspace(msa.msa_sparse_attn_workspace_size(1, 1, T, Hq, Hkv, M, T))
    msa.msa_sparse_attn_lse(ctx128, dev["Q"], dev["KV"], mo, M, dev["Kl"], dev["Vl"], qoff, W.scale_of(d), O, lse, ws)
    g_ = [torch.empty_like(dev[k]) for k in ("Q", "KV", "Kl", "Vl")]
    wsb = msa.workspace(msa.msa_sparse_attn_bwd_workspace_size(1, 1, T, Hq, Hkv, M, T))
    msa.msa_sparse_attn_bwd(ctx128, dev["Q"], dev["KV"], mo, M, dev["Kl"], dev["Vl"], qoff, W.scale_of(d), O,
                            dev["dO"], lse, *g_, wsb)
    torch.cuda.synchronize()
    dQ, dKV, dKl, dVl = (W.widen(W.host_bits(t), "bf16") for t in g_)

    host = {k: W.widen(W.counter_bf16_threads(seed, streams[k], 0, int(np.prod(shp))).reshape(shp), "bf16")
            for k, shp in shapes.items()}
    g = 5
    G = Hq // Hkv
    q_rows = np.concatenate([np.arange(8), [1000, 4095, 4096, 4097, 6001], np.arange(T - 27, T)])
    key_rows = np.concatenate([[0, 1, 100, 240, 241], np.arange(242, 250), [242 + 31, 242 + 32, 4000, 8191],
                               np.arange(M + T - 30, M + T)])
    rq, rk, rv = oracle.sparse_attn_bwd_sampled(host["Q"][0], host["KV"][:, 0], host["KV"][:, 1], host["Kl"][0],
                                                host["Vl"][0], qoff, W.scale_of(d), ctx128.rope_theta,
                                                host["dO"][0], g, q_rows, key_rows)
    got_q = dQ[0][q_rows][:, g * G:(g + 1) * G]
    allk = np.concatenate([dKV[:, 0, g], dKl[0, :, g]])
    allv = np.concatenate([dKV[:, 1, g], dVl[0, :, g]])
    for name, got, ref in (("dQ", got_q, rq), ("dK", allk[key_rows], rk), ("dV", allv[key_rows], rv)):
        print(f"\n{name}: rel max err {_rel(got, ref):.3e}", flush=True)
        assert _rel(got, ref) <= GRAD_TOL, name


ENC_CASES = [
    # dtype, d, Hkv, chunk_len, document lengths
    ("f32", 64, 2, 16, [256] * 64),                          # the tiny fp32 bank
    ("bf16", 128, 8, 64, list(range(128, 1024, 37))),       # Qwen-shaped, ragged last chunks
    ("bf16", 128, 8, 5, [1, 2, 5, 6, 13, 4, 9]),            # short documents, partial chunks
    ("f32", 128, 4, 1, [3, 1, 7]),                           # chunk 1: one row per token
]


@pytest.mark.parametrize("dtype,d,Hkv,chunk_len,lens", ENC_CASES)
def test_encode_pool_bwd_parity(torch_mod, msa, ctx64, ctx128, dtype, d, Hkv, chunk_len, lens):
    torch = torch_mod
    ctx = ctx128 if d == 128 else ctx64
    tok = msa_synth.prefix_offsets(lens)
    coff = msa_synth.prefix_offsets([(n + chunk_len - 1) // chunk_len for n in lens])
    T, N = int(tok[-1]), int(coff[-1])
    gKV = W.draw(111, 1, (N, 2, Hkv, d), dtype)
    gR = W.draw(111, 2, (N, Hkv, d), dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = [torch.full((T, Hkv, d), float("nan"), dtype=tdt, device="cuda") for _ in range(3)]
    msa.msa_encode_pool_bwd(ctx, W.dev(gKV, dtype), W.dev(gR, dtype), torch.from_numpy(tok).cuda(),
                            torch.from_numpy(coff).cuda(), *out, chunk_len, max(lens))
    torch.cuda.synchronize()
    g = W.widen(gKV, dtype)
    ref = oracle.encode_pool_bwd(g[:, 0], g[:, 1], W.widen(gR, dtype), tok, chunk_len, ctx.rope_theta)
    tol = 2e-2 if dtype == "bf16" else 1e-5
    for name, t, r in zip(("dK", "dV", "dKr"), out, ref):
        got = W.widen(W.host_bits(t), dtype)
        assert np.all(np.isfinite(got)), name
        assert W.rel_row_err(got, r) <= tol, (name, W.rel_row_err(got, r))


def test_backward_validation_errors(torch_mod, msa, ctx128):
    """Bad arguments are refused before anything is enqueued."""
    torch = torch_mod
    x = _inputs(121, "bf16", 128, 32, 8, 1, 8, 16, [4])
    dev = {k: W.dev_bf16(x[k]) for k in ("Q", "KV", "Kl", "Vl", "dO")}
    mo = torch.tensor([0, 4], dtype=torch.int64, device="cuda")
    O = torch.empty_like(dev["Q"])
    lse = torch.empty((1, 8, 32), dtype=torch.float32, device="cuda")
    ws_f = msa.workspace(msa.msa_sparse_attn_workspace_size(1, 1, 8, 32, 8, 4, 16))
    with pytest.raises(msa.MsaError) as e:                       # lse missing
        msa.msa_sparse_attn_lse(ctx128, dev["Q"], dev["KV"], mo, 4, dev["Kl"], dev["Vl"], 16, 0.088, O, None, ws_f)
    assert e.value.status == msa.MSA_ERR_INVALID_ARG
    msa.msa_sparse_attn_lse(ctx128, dev["Q"], dev["KV"], mo, 4, dev["Kl"], dev["Vl"], 16, 0.088, O, lse, ws_f)
    g = [torch.empty_like(dev[k]) for k in ("Q", "KV", "Kl", "Vl")]
    need = msa.msa_sparse_attn_bwd_workspace_size(1, 1, 8, 32, 8, 4, 16)
    small = msa.workspace(need - 256)
    with pytest.raises(msa.MsaError) as e:                       # workspace too small
        msa.msa_sparse_attn_bwd(ctx128, dev["Q"], dev["KV"], mo, 4, dev["Kl"], dev["Vl"], 16, 0.088, O, dev["dO"],
                                lse, *g, small)
    assert e.value.status == msa.MSA_ERR_WORKSPACE
    ws = msa.workspace(need)
    with pytest.raises(msa.MsaError) as e:                       # Tq > L
        msa.msa_sparse_attn_bwd(ctx128, dev["Q"], dev["KV"], mo, 4, dev["Kl"][:, :4].contiguous(),
                                dev["Vl"][:, :4].contiguous(), 16, 0.088, O, dev["dO"], lse, g[0], g[1],
                                g[2][:, :4].contiguous(), g[3][:, :4].contiguous(), ws)
    assert e.value.status == msa.MSA_ERR_INVALID_ARG
    with pytest.raises(msa.MsaError) as e:                       # dO missing
        msa.msa_sparse_attn_bwd(ctx128, dev["Q"], dev["KV"], mo, 4, dev["Kl"], dev["Vl"], 16, 0.088, O, None,
                                lse, *g, ws)
    assert e.value.status == msa.MSA_ERR_INVALID_ARG
    # pooling backward: more chunk rows than tokens
    gkv = torch.zeros((10, 2, 8, 128), dtype=torch.bfloat16, device="cuda")
    gr = torch.zeros((10, 8, 128), dtype=torch.bfloat16, device="cuda")
    out = [torch.empty((5, 8, 128), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    tok = torch.tensor([0, 5], dtype=torch.int64, device="cuda")
    coff = torch.tensor([0, 10], dtype=torch.int64, device="cuda")
    with pytest.raises(msa.MsaError) as e:
        msa.msa_encode_pool_bwd(ctx128, gkv, gr, tok, coff, *out, 1, 5)
    assert e.value.status == msa.MSA_ERR_INVALID_ARG
    torch.cuda.synchronize()
