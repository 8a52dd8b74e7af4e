"""Route once, then generate: the pages' inference pipeline end to end on a
reduced bank (GPU only), through the C ABI.

neo-ai.one MSA article, 推論パイプライン (Fig. 3), and the ruixiangma.github.io
blog, 三阶段推理流程: the documents are selected once, when the context is
assembled, and generation then attends over the same gathered K̄/V̄ plus a
local context that grows by one token per generated token.

Assembly runs as the route-once workload runs it: layer l+1's routing is
enqueued before the host takes layer l's ids, and msa_gather copies layer l's
documents with hipMemcpyAsync on a side stream while that routing runs.
Generation: four tokens, each attending in every one of three layers.
Checked against the oracle: every layer's top-16 (a planted set, bit-exact),
the gathered rows (byte-exact, in ascending document order) and the output
of every (token, layer) pair at the attention bar (2e-2, absolute and
relative to max|O_ref|).  Memory rows of the planted documents and each
token's own local key are aimed at that token's query (tests/peaked.py), so
the softmax is peaked and a wrong position, a stale or missing row or a
wrong local length moves the output by far more than the bar.
"""

import math

import numpy as np
import pytest

import msa_synth
import oracle
from tests import peaked as P
from tests import workloads as W

pytestmark = pytest.mark.gpu

Hq, Hkv, D, C = 32, 8, 128, 64
G = Hq // Hkv
LAYERS, K, L0, T = 3, 16, 300, 4
THETA = 1e6
SEED = 61


def _bits(x64):
    return oracle.f64_to_bf16_bits(x64)


@pytest.fixture(scope="module")
def bank():
    """Inputs of every layer, built on the host: bf16 bits and the offsets."""
    lens = msa_synth.lognormal_lengths(SEED, 200_000)
    coff = msa_synth.ceil_chunk_offsets(lens, C)
    n_docs, N = len(lens), int(coff[-1])
    planted = msa_synth.pick_planted(SEED, 50, n_docs, K)
    layers = []
    for l in range(LAYERS):
        Qr = msa_synth.normal_bf16(SEED, 100 + l, (1, 1, Hq, D))
        Kr = msa_synth.normal_bf16(SEED, 110 + l, (N, Hkv, D))
        q = msa_synth.bf16_bits_to_f32(Qr)[0, 0]
        for j, d in enumerate(planted):
            Kr[coff[d]:coff[d + 1]] = W.planted_pooled(SEED, l, q, Hkv, int(coff[d + 1] - coff[d]), tag=j)
        Q = [msa_synth.normal_bf16(SEED, 200 + 10 * l + t, (1, 1, Hq, D)) for t in range(T)]
        q64 = [oracle.bf16_bits_to_f64(x)[0, 0] for x in Q]
        kv = oracle.bf16_bits_to_f64(msa_synth.normal_bf16(SEED, 120 + l, (N, 2, Hkv, D)))
        kv[:, 1] *= P.V_SCALE
        for t in range(T):                # token t's memory keys: the first row of planted docs t, t+T, ...
            keys = P.aim_memory_keys(q64[t], K + L0 + t, THETA, G)
            for d in planted[t::T]:
                kv[coff[d], 0] = keys
        kl = oracle.bf16_bits_to_f64(msa_synth.normal_bf16(SEED, 130 + l, (1, L0 + T, Hkv, D)))
        vl = P.V_SCALE * oracle.bf16_bits_to_f64(msa_synth.normal_bf16(SEED, 140 + l, (1, L0 + T, Hkv, D)))
        for t in range(T):                # token t's own local key
            kl[0, L0 + t] = P.aim_local_keys(q64[t], 0, THETA, G)
        layers.append(dict(Qr=Qr, Kr=Kr, Q=Q, KV=_bits(kv), Kl=_bits(kl), Vl=_bits(vl)))
    return dict(lens=lens, coff=coff, n_docs=n_docs, N=N, planted=planted, layers=layers)


def test_route_once_then_generate(gpu, bank):
    import torch
    import long_context_memory_chunk_amd as msa
    msa.lib()
    ctx = msa.msa_ctx_create(0, D, THETA, 16384)
    coff, N, n_docs = bank["coff"], bank["N"], bank["n_docs"]
    lay = bank["layers"]
    coff_dev = torch.from_numpy(coff).cuda()
    cap = int(np.sort(np.diff(coff))[-K:].sum())
    host = []
    for l in range(LAYERS):
        h = torch.empty((N, 2, Hkv, D), dtype=torch.bfloat16, pin_memory=True)
        h.view(torch.int16).numpy()[:] = lay[l]["KV"].view(np.int16)
        host.append(h)
    Kr = [W.dev_bf16(x["Kr"]) for x in lay]
    Qr = [W.dev_bf16(x["Qr"]) for x in lay]
    ws_r = [msa.workspace(msa.msa_route_workspace_size(1, 1, 1, Hq, Hkv, N, n_docs, K)) for _ in range(2)]
    ids_h = torch.empty((LAYERS, 1, K), dtype=torch.int32, pin_memory=True)
    ids_np = [ids_h[l].numpy() for l in range(LAYERS)]
    KVmem = torch.full((LAYERS, cap, 2, Hkv, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    mo_h = torch.zeros((LAYERS, 2), dtype=torch.int64, pin_memory=True)
    mo_d = torch.zeros((LAYERS, 2), dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    ev = [torch.cuda.Event() for _ in range(LAYERS)]

    # ---- assembly: route layer l+1 while layer l's documents are copied
    msa.msa_route(ctx, Qr[0], Kr[0], coff_dev, K, ids_h[0], ws_r[0])
    ev[0].record(main)
    for l in range(LAYERS):
        if l + 1 < LAYERS:
            msa.msa_route(ctx, Qr[l + 1], Kr[l + 1], coff_dev, K, ids_h[l + 1], ws_r[(l + 1) % 2])
            ev[l + 1].record(main)
        ev[l].synchronize()
        msa.msa_gather(host[l], 2 * Hkv * D * 2, N, coff, ids_np[l], K, KVmem[l], cap, mo_h[l], mo_d[l],
                       side=side)
    main.wait_stream(side)

    # ---- generation: T tokens, each through every layer, local context growing by one
    Kl = [W.dev_bf16(x["Kl"]) for x in lay]
    Vl = [W.dev_bf16(x["Vl"]) for x in lay]
    Qd = [[W.dev_bf16(x["Q"][t]) for x in lay] for t in range(T)]
    O = torch.full((T, LAYERS, 1, 1, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws_a = msa.workspace(msa.msa_sparse_attn_workspace_size(1, 1, 1, Hq, Hkv, cap, L0 + T))
    scale = 1.0 / math.sqrt(D)
    for t in range(T):
        for l in range(LAYERS):
            n = L0 + t + 1
            msa.msa_sparse_attn(ctx, Qd[t][l], KVmem[l], mo_d[l], cap, Kl[l][:, :n], Vl[l][:, :n], K, scale,
                                O[t, l], ws_a)
    torch.cuda.synchronize()

    # ---- the oracle, layer by layer
    got_O = W.widen(W.host_bits(O), "bf16")
    planted = sorted(int(d) for d in bank["planted"])
    for l in range(LAYERS):
        ids_ref, sc_ref, _, D_ref = oracle.route(W.widen(lay[l]["Qr"], "bf16"), W.widen(lay[l]["Kr"], "bf16"),
                                                 coff, K)
        assert sorted(ids_np[l][0].tolist()) == sorted(ids_ref[0].tolist()) == planted, l
        assert sc_ref[0].min() - np.delete(D_ref[0], ids_ref[0]).max() >= 0.05
        rows, m = oracle.gather_rows(lay[l]["KV"], coff, ids_ref[0])
        assert mo_h[l].tolist() == [0, m] and mo_d[l].cpu().tolist() == [0, m]
        assert np.array_equal(W.host_bits(KVmem[l, :m]), rows), f"layer {l}: gathered rows"
        kv = W.widen(rows, "bf16")
        for t in range(T):
            n = L0 + t + 1
            ref = oracle.sparse_attn(W.widen(lay[l]["Q"][t], "bf16"), kv[:, 0], kv[:, 1], [0, m],
                                     W.widen(lay[l]["Kl"][:, :n], "bf16"), W.widen(lay[l]["Vl"][:, :n], "bf16"),
                                     K, scale, THETA)
            assert np.max(np.abs(ref)) > 0.25
            P.assert_attn_close(got_O[t, l], ref, 2e-2, f"route-once layer {l} token {t}")
    ctx.close()
