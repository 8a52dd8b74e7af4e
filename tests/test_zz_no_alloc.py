"""msa_sparse_attn_noalloc (the attention call without a workspace, for
callers that cannot allocate) against msa_sparse_attn with a workspace, through
the C ABI (GPU only).

Both run the same kernels with the same launch plan, so the outputs must be
bit-identical; both are also held to the attention bar against the oracle
(2e-2 bf16, 1e-3 fp32, absolute and relative to max|O_ref|).  Two calls in a
row share the library's scratch array, the second with a smaller input, so
leftovers of the first call must not leak into the second.
"""

import numpy as np
import pytest

import oracle
from tests import peaked as P
from tests import workloads as W

pytestmark = pytest.mark.gpu

SCRATCH = 16 << 20


@pytest.fixture(scope="module")
def env(gpu):
    import torch
    import long_context_memory_chunk_amd as msa
    msa.lib()
    ctx = msa.msa_ctx_create(0, 128, P.THETA, 16384)
    yield torch, msa, ctx
    ctx.close()


def _both(torch, msa, ctx, w, dtype):
    B, Tq, Hq, D = w["Q"].shape
    L, Hkv = w["Kl"].shape[1], w["Kl"].shape[2]
    max_rows = max(int(np.diff(w["mem_off"]).max()), 1)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def put(bits):
        return W.dev_bf16(bits) if dtype == "bf16" else W.dev_f32(oracle.bf16_bits_to_f64(bits))

    Q, KV, Kl, Vl = (put(w[k]) for k in ("Q", "KV", "Kl", "Vl"))
    mo = torch.from_numpy(w["mem_off"]).cuda()
    O_ws = torch.full((B, Tq, Hq, D), float("nan"), dtype=tdt, device="cuda")
    O_na = torch.full_like(O_ws, float("nan"))
    dt = 1 if dtype == "bf16" else 0
    need = msa.msa_sparse_attn_workspace_size(dt, B, Tq, Hq, Hkv, max_rows, L)
    assert need <= SCRATCH
    ws = msa.workspace(need)
    msa.msa_sparse_attn(ctx, Q, KV, mo, max_rows, Kl, Vl, w["qoff"], w["scale"], O_ws, ws)
    msa.msa_sparse_attn_noalloc(ctx, Q, KV, mo, max_rows, Kl, Vl, w["qoff"], w["scale"], O_na)
    torch.cuda.synchronize()
    return W.host_bits(O_ws), W.host_bits(O_na)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_the_workspace_call_twice_second_smaller(env, dtype):
    torch, msa, ctx = env
    tol = 2e-2 if dtype == "bf16" else 1e-3
    big = P.peaked_inputs(51, 4, 2, 32, 8, 128, 2048, [300, 0, 1000, 64], 16, P.THETA, tokens=[0, 1])
    small = P.peaked_inputs(52, 1, 1, 32, 8, 128, 300, [40], 16, P.THETA)
    for name, w in (("first, larger", big), ("second, smaller", small)):
        ws_bits, na_bits = _both(torch, msa, ctx, w, dtype)
        assert np.array_equal(ws_bits, na_bits), name
        P.assert_attn_close(W.widen(na_bits, dtype), P.oracle_out(w), tol, f"noalloc {dtype} {name}")


def test_noalloc_short_prefill_on_the_matrix_cores(env):
    """A 256-token query block (the matrix-core prefill kernel, whose packed
    key tiles also live in the scratch) then a decode."""
    torch, msa, ctx = env
    pre = P.peaked_inputs(53, 1, 256, 32, 8, 128, 512, [200], 16, P.THETA, tokens=[0, 255])
    dec = P.peaked_inputs(54, 2, 1, 32, 8, 128, 700, [90, 10], 16, P.THETA)
    for name, w in (("prefill", pre), ("decode after prefill", dec)):
        ws_bits, na_bits = _both(torch, msa, ctx, w, "bf16")
        assert np.array_equal(ws_bits, na_bits), name
        P.assert_attn_close(W.widen(na_bits, "bf16"), P.oracle_out(w), 2e-2, f"noalloc {name}")


def test_noalloc_refuses_a_call_beyond_the_scratch(env):
    torch, msa, ctx = env
    B, Tq, L, rows = 1, 8192, 8192, 250         # the 8K prefill's packed key tiles exceed the scratch
    assert msa.msa_sparse_attn_workspace_size(1, B, Tq, 32, 8, rows, L) > SCRATCH
    Q = torch.zeros((B, Tq, 32, 128), dtype=torch.bfloat16, device="cuda")
    KV = torch.zeros((rows, 2, 8, 128), dtype=torch.bfloat16, device="cuda")
    Kl = torch.zeros((B, L, 8, 128), dtype=torch.bfloat16, device="cuda")
    mo = torch.tensor([0, rows], dtype=torch.int64, device="cuda")
    O = torch.zeros_like(Q)
    with pytest.raises(msa.MsaError) as e:
        msa.msa_sparse_attn_noalloc(ctx, Q, KV, mo, rows, Kl, Kl, 16, 0.088, O)
    assert e.value.status == msa.MSA_ERR_WORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
