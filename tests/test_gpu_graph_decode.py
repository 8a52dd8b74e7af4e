"""The generation step under HIP graph capture (GPU only), through the C ABI.

A token-by-token generation loop attends in every layer over the rows
gathered at context assembly and a local context one token longer each step
(neo-ai.one MSA article, 推論パイプライン, Fig. 3, third stage).  Such a loop
is captured once per token position and replayed; msa_sparse_attn_noalloc
needs no workspace, so the captured calls allocate nothing.  Every replay,
with eager calls and synchronisations of the program between replays, must
give the eager result bit for bit, and the eager result matches the oracle.
"""

import math

import numpy as np
import pytest

import oracle
from tests import peaked as P
from tests import workloads as W

pytestmark = pytest.mark.gpu

Hq, Hkv, D, LAYERS, K, L0, T = 32, 8, 128, 3, 16, 400, 3


def test_generation_graphs_replay_bit_exact(gpu):
    import torch
    import long_context_memory_chunk_amd as msa
    msa.lib()
    ctx = msa.msa_ctx_create(0, D, P.THETA, 16384)
    rows = [150, 90, 200]
    ins = [P.peaked_inputs(70 + l, 1, 1, Hq, Hkv, D, L0 + T, [rows[l]], K, P.THETA) for l in range(LAYERS)]
    KV = [W.dev_bf16(w["KV"]) for w in ins]
    mo = [torch.from_numpy(w["mem_off"]).cuda() for w in ins]
    Kl = [W.dev_bf16(w["Kl"]) for w in ins]
    Vl = [W.dev_bf16(w["Vl"]) for w in ins]
    Q = [[W.dev_bf16(np.ascontiguousarray(np.roll(w["Q"], t, axis=-1))) for w in ins] for t in range(T)]
    scale = 1.0 / math.sqrt(D)

    def token(t, out):
        for l in range(LAYERS):
            n = L0 + t + 1
            msa.msa_sparse_attn_noalloc(ctx, Q[t][l], KV[l], mo[l], rows[l], Kl[l][:, :n], Vl[l][:, :n], K, scale,
                                        out[l])

    eager = [[torch.empty((1, 1, Hq, D), dtype=torch.bfloat16, device="cuda") for _ in range(LAYERS)]
             for _ in range(T)]
    for t in range(T):
        token(t, eager[t])
    torch.cuda.synchronize()
    ref_bits = [[W.host_bits(x) for x in e] for e in eager]

    graphs, outs = [], []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for t in range(T):
            out = [torch.full((1, 1, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
                   for _ in range(LAYERS)]
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                token(t, out)
            graphs.append(g)
            outs.append(out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    other = [torch.empty((1, 1, Hq, D), dtype=torch.bfloat16, device="cuda") for _ in range(LAYERS)]
    for rep in range(3):
        for t in range(T):
            for x in outs[t]:
                x.fill_(float("nan"))
            graphs[t].replay()
            token((t + 1) % T, other)              # the program's own eager work between replays
            torch.cuda.synchronize()
            for l in range(LAYERS):
                assert np.array_equal(W.host_bits(outs[t][l]), ref_bits[t][l]), (rep, t, l)

    # the eager result itself against the oracle
    for t in range(T):
        for l in range(LAYERS):
            w = ins[l]
            n = L0 + t + 1
            kv = oracle.bf16_bits_to_f64(w["KV"])
            ref = oracle.sparse_attn(oracle.bf16_bits_to_f64(np.roll(w["Q"], t, axis=-1)), kv[:, 0], kv[:, 1],
                                     w["mem_off"], oracle.bf16_bits_to_f64(w["Kl"][:, :n]),
                                     oracle.bf16_bits_to_f64(w["Vl"][:, :n]), K, scale, P.THETA)
            P.assert_attn_close(W.widen(ref_bits[t][l], "bf16"), ref, 2e-2, f"graph layer {l} token {t}")
    del graphs
    ctx.close()
