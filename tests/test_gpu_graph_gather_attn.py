"""msa_gather_attn under HIP graph capture (GPU only), through the C ABI.

A decode loop may capture its per-layer calls and replay them.  The call's
launches (the gather plan, the copy beside the local keys' attention, the
memory rows' attention, the merge) clear nothing with memset and allocate
nothing, so a captured layer must give, on every replay, with eager calls and
synchronisations of the program between replays, the eager result bit for
bit: the gathered rows, their offsets and the attention output.  The eager
result itself is checked against the oracle (neo-ai.one MSA article,
推論パイプライン, Fig. 3: the selected K̄/V̄ loaded and concatenated with the
local context).
"""

import numpy as np
import pytest

import oracle
from tests import peaked as P
from tests import workloads as W
from tests.test_gpu_gather_attn import _bank

pytestmark = pytest.mark.gpu

D = 128


def test_gather_attn_graph_replay_bit_exact(gpu):
    import torch
    import long_context_memory_chunk_amd as msa
    msa.lib()
    ctx = msa.msa_ctx_create(0, D, P.THETA, 16384)
    # (seed, B, rows per query, top_k): the bounded copy with its plan, and the one-query copy
    layers = [(81, 4, [120, 0, 45, 200], 8), (82, 1, [130], 16)]
    Hq, Hkv, L = 32, 8, 512
    setup = []
    for seed, B, rows, k in layers:
        w = P.peaked_inputs(seed, B, 1, Hq, Hkv, D, L, rows, k, P.THETA)
        bank, coff, ids = _bank(w, k, seed)
        host = torch.empty(bank.shape, dtype=torch.bfloat16, pin_memory=True)
        host.copy_(W.dev_bf16(bank, "cpu"))
        cap = int(sum(rows))
        max_rows = max(rows)
        ws = msa.workspace(msa.msa_gather_attn_workspace_size(1, B, 1, Hq, Hkv, k, cap, max_rows, L))
        setup.append(dict(w=w, bank=bank, coff=coff, ids=ids, host=host, B=B, k=k, cap=cap, max_rows=max_rows,
                          coff_d=torch.from_numpy(coff).cuda(), ids_d=torch.from_numpy(ids).cuda(),
                          Q=W.dev_bf16(w["Q"]), Kl=W.dev_bf16(w["Kl"]), Vl=W.dev_bf16(w["Vl"]), ws=ws))

    def outputs(c):
        return (torch.full((max(c["cap"], 1), 2, Hkv, D), float("nan"), dtype=torch.bfloat16, device="cuda"),
                torch.full((c["B"] + 1,), -7, dtype=torch.int64, device="cuda"),
                torch.full((c["B"], 1, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda"))

    def call(c, out):
        dst, mo, O = out
        msa.msa_gather_attn(ctx, c["host"], 2 * Hkv * D * 2, c["bank"].shape[0], c["coff_d"], c["ids_d"], dst,
                            c["cap"], mo, c["Q"], c["max_rows"], c["Kl"], c["Vl"], c["k"], c["w"]["scale"], O,
                            c["ws"])

    eager = [outputs(c) for c in setup]
    for c, out in zip(setup, eager):
        call(c, out)
    torch.cuda.synchronize()
    ref = [[W.host_bits(out[0]), out[1].cpu().numpy(), W.host_bits(out[2])] for out in eager]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    outs = [outputs(c) for c in setup]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for c, out in zip(setup, outs):
                call(c, out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    other = [outputs(c) for c in setup]
    for rep in range(3):
        for out in outs:
            out[0].fill_(float("nan"))
            out[1].fill_(-7)
            out[2].fill_(float("nan"))
        g.replay()
        for c, o in zip(setup, other):       # the program's own eager calls between replays
            call(c, o)
        torch.cuda.synchronize()
        for i, out in enumerate(outs):
            n = int(ref[i][1][-1])
            assert np.array_equal(out[1].cpu().numpy(), ref[i][1]), (rep, i)
            assert np.array_equal(W.host_bits(out[0])[:n], ref[i][0][:n]), (rep, i)
            assert np.array_equal(W.host_bits(out[2]), ref[i][2]), (rep, i)

    # the eager result against the oracle
    for i, c in enumerate(setup):
        w = c["w"]
        assert np.array_equal(ref[i][1], np.asarray(w["mem_off"], dtype=np.int64))
        for b in range(c["B"]):
            rows_b, _ = oracle.gather_rows(c["bank"], c["coff"], c["ids"][b])
            assert np.array_equal(ref[i][0][ref[i][1][b]:ref[i][1][b + 1]], rows_b)
        P.assert_attn_close(W.widen(ref[i][2], "bf16"), P.oracle_out(w), 2e-2, f"graph gather_attn layer {i}")
    del g
    ctx.close()
