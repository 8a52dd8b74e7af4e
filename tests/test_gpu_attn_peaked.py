"""Attention parity on peaked inputs (GPU only), through the C ABI.

The inputs of tests/peaked.py plant, for each checked query token, memory
rows and local keys that carry most of the softmax mass, so |O| is of order
one and the output moves by far more than the bar if the kernel shifts the
global RoPE offset k by a position, drops memory rows, skips the token's own
key or reads a row range one row late (tests/test_oracle_attention_controls.py
shows each of those mistakes failing the bar on these same inputs).  The bar:
max|O - O_ref| <= tol and <= tol * max|O_ref|, tol 2e-2 in bf16 and 1e-3 in
fp32 (neo-ai.one MSA article, 全体設計 › アーキテクチャ: memory rows before
the local context, global RoPE shifted by k, causal local keys).
"""

import numpy as np
import pytest

import oracle
from tests import peaked as P
from tests import workloads as W

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module")
def env(gpu):
    import torch
    import long_context_memory_chunk_amd as msa
    msa.lib()
    ctx = msa.msa_ctx_create(0, D, P.THETA, 16384)
    yield torch, msa, ctx
    ctx.close()


def _run(torch, msa, ctx, w, dtype="bf16"):
    B, Tq, Hq, _ = w["Q"].shape
    L, Hkv = w["Kl"].shape[1], w["Kl"].shape[2]
    rows = np.diff(w["mem_off"])
    max_rows = max(int(rows.max()), 1)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def put(bits):
        return W.dev_bf16(bits) if dtype == "bf16" else W.dev_f32(oracle.bf16_bits_to_f64(bits))

    O = torch.full((B, Tq, Hq, D), float("nan"), dtype=tdt, device="cuda")
    ws = msa.workspace(msa.msa_sparse_attn_workspace_size(1 if dtype == "bf16" else 0, B, Tq, Hq, Hkv,
                                                          max_rows, L))
    msa.msa_sparse_attn(ctx, put(w["Q"]), put(w["KV"]), torch.from_numpy(w["mem_off"]).cuda(), max_rows,
                        put(w["Kl"]), put(w["Vl"]), w["qoff"], w["scale"], O, ws)
    torch.cuda.synchronize()
    return W.widen(W.host_bits(O), dtype)


@pytest.mark.parametrize("seed,B,Tq,Hq,Hkv,L,rows,qoff", P.DECODE_CASES)
def test_peaked_decode(env, seed, B, Tq, Hq, Hkv, L, rows, qoff):
    torch, msa, ctx = env
    w = P.peaked_inputs(seed, B, Tq, Hq, Hkv, D, L, rows, qoff, P.THETA, tokens=list(range(Tq)))
    got = _run(torch, msa, ctx, w)
    ref = P.oracle_out(w)
    assert np.max(np.abs(ref)) > 0.25
    P.assert_attn_close(got, ref, 2e-2, f"decode B={B} Tq={Tq} G={Hq // Hkv} L={L} rows={rows}")


@pytest.mark.parametrize("seed,B,Tq,Hq,Hkv,L,rows,qoff", P.DECODE_CASES)
def test_peaked_decode_closest_to_its_own_offset(env, seed, B, Tq, Hq, Hkv, L, rows, qoff):
    """Negative control on the GPU output itself: it sits closer to the oracle
    at the global RoPE offset k it was called with than to the oracle at k - 1
    or k + 1, or with every query's memory range read one row late."""
    torch, msa, ctx = env
    w = P.peaked_inputs(seed, B, Tq, Hq, Hkv, D, L, rows, qoff, P.THETA, tokens=list(range(Tq)))
    got = _run(torch, msa, ctx, w)
    dist = lambda ref: float(np.max(np.abs(got - ref)))
    own = dist(P.oracle_out(w))
    wrong = {"k+1": P.oracle_out(w, qoff=qoff + 1), "late": P.oracle_out(w, mem_late=True)}
    if qoff > 0:
        wrong["k-1"] = P.oracle_out(w, qoff=qoff - 1)
    for name, ref in wrong.items():
        print(f"[attn] distance to the oracle at k {own:.3e}, to {name} {dist(ref):.3e}", flush=True)
        assert own < dist(ref), name


def test_peaked_decode_fp32(env):
    """The same planted decode in fp32 (the vector-unit kernel), bar 1e-3."""
    torch, msa, ctx = env
    seed, B, Tq, Hq, Hkv, L, rows, qoff = P.DECODE_CASES[2]
    w = P.peaked_inputs(seed, B, Tq, Hq, Hkv, D, L, rows, qoff, P.THETA)
    got = _run(torch, msa, ctx, w, dtype="f32")
    P.assert_attn_close(got, P.oracle_out(w), 1e-3, "decode fp32")


@pytest.mark.parametrize("B,Tq,L,rows,tokens", [
    (2, 256, 600, [250, 90], [0, 100, 255]),     # query block on the matrix cores, full output checked
    (1, 200, 200, [130], [7, 128, 199]),          # Tq = L, ragged query tile
])
def test_peaked_prefill_full_output(env, B, Tq, L, rows, tokens):
    torch, msa, ctx = env
    w = P.peaked_inputs(41, B, Tq, 32, 8, D, L, rows, 32, P.THETA, tokens=tokens)
    got = _run(torch, msa, ctx, w)
    ref = P.oracle_out(w)
    P.assert_attn_close(got, ref, 2e-2, f"prefill B={B} Tq={Tq} L={L}")
    for i in tokens:          # the planted tokens are the peaked rows; check them on their own too
        P.assert_attn_close(got[:, i], ref[:, i], 2e-2, f"prefill token {i}")


@pytest.mark.timeout(600)
def test_peaked_prefill_8k_sampled_tokens(env):
    """Causal prefill of 8,192 tokens over 250 memory rows, launched as the
    prefill workload launches it; tokens 4095 and 8191 are planted, and those
    plus unplanted tokens are checked against the oracle one by one."""
    torch, msa, ctx = env
    c = P.PREFILL_CASE
    w = P.peaked_inputs(c["seed"], 1, c["T"], 32, 8, D, c["T"], [c["M"]], c["qoff"], P.THETA,
                        tokens=c["tokens"])
    got = _run(torch, msa, ctx, w)
    for i in (*c["tokens"], 0, 1, 127, 128, 4094, 6000):
        ref = P.oracle_out(P.token_view(w, i))
        if i in c["tokens"]:
            assert np.max(np.abs(ref)) > 0.25
        P.assert_attn_close(got[:, i:i + 1], ref, 2e-2, f"8K prefill token {i}")
