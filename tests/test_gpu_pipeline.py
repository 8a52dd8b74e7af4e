"""End-to-end: encode -> route -> gather (pinned host store) -> sparse attention,
through the C ABI, against the oracle run on its own from the same seeded
inputs (GPU only).  Tolerances as in test_gpu_parity.py."""

import numpy as np
import pytest

import msa_synth
import oracle
from tests import peaked as P
from tests import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa(gpu):
    import long_context_memory_chunk_amd as m
    m.lib()
    return m


def _gather_and_attend(torch, msa, ctx, KVbar, coff, ids, Q, Kl, Vl, top_k, dtype):
    """Product flow after routing: bank to pinned host memory, gather the
    selected documents back, attend."""
    N = KVbar.shape[0]
    host = torch.empty(KVbar.shape, dtype=KVbar.dtype, pin_memory=True)
    host.copy_(KVbar)
    row_bytes = KVbar[0].numel() * KVbar.element_size()
    cap = int(np.sum(np.diff(coff)[ids.reshape(-1)]))
    dst = torch.empty((max(cap, 1),) + tuple(KVbar.shape[1:]), dtype=KVbar.dtype, device="cuda")
    mo_host = torch.zeros(ids.shape[0] + 1, dtype=torch.int64, pin_memory=True)
    mo_dev = torch.zeros(ids.shape[0] + 1, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    msa.msa_gather(host, row_bytes, N, coff, np.ascontiguousarray(ids, dtype=np.int32), top_k, dst,
                   cap, mo_host, mo_dev, side=side)
    torch.cuda.current_stream().wait_stream(side)
    B, Tq, Hq, d = Q.shape
    Hkv = Kl.shape[2]
    max_rows = int(np.max(np.diff(mo_host.numpy())))
    ws = msa.workspace(msa.msa_sparse_attn_workspace_size(1 if dtype == "bf16" else 0, B, Tq, Hq, Hkv,
                                                          max_rows, Kl.shape[1]))
    O = torch.empty(Q.shape, dtype=Q.dtype, device="cuda")
    msa.msa_sparse_attn(ctx, Q, dst, mo_dev, max_rows, Kl, Vl, top_k, W.scale_of(d), O, ws)
    torch.cuda.synchronize()
    return O


def test_tiny_fp32_end_to_end(gpu, msa):
    import torch
    w = W.tiny_fp32()
    ctx = msa.msa_ctx_create(0, w["d"], w["theta"], 4096)
    tok = w["tok_off"]
    coff, max_len = msa.msa_chunk_offsets(tok, w["chunk"], with_max_len=True)
    N = int(coff[-1])
    KVbar = torch.empty((N, 2, w["Hkv"], w["d"]), dtype=torch.float32, device="cuda")
    Krbar = torch.empty((N, w["Hkv"], w["d"]), dtype=torch.float32, device="cuda")
    msa.msa_encode_pool(ctx, W.dev_f32(w["K"]), W.dev_f32(w["V"]), W.dev_f32(w["Kr"]),
                        torch.from_numpy(tok).cuda(), torch.from_numpy(coff).cuda(), KVbar, Krbar,
                        w["chunk"], max_len)
    ids = torch.empty((1, w["top_k"]), dtype=torch.int32, device="cuda")
    ws = msa.workspace(msa.msa_route_workspace_size(0, 1, w["Tq"], w["Hq"], w["Hkv"], N, 64, w["top_k"]))
    msa.msa_route(ctx, W.dev_f32(w["Qr"]), Krbar, torch.from_numpy(coff).cuda(), w["top_k"], ids, ws)
    ids_h = ids.cpu().numpy()
    O = _gather_and_attend(torch, msa, ctx, KVbar, coff, ids_h, W.dev_f32(w["Q"]), W.dev_f32(w["K_loc"]),
                           W.dev_f32(w["V_loc"]), w["top_k"], "f32")

    Kb, Vb, Rb = oracle.encode_pool(w["K"], w["V"], w["Kr"], tok, w["chunk"], w["theta"])
    Kb, Vb, Rb = (W.round_store(x, "f32") for x in (Kb, Vb, Rb))
    ids_ref, sc_ref, _, D_ref = oracle.route(w["Qr"].astype(np.float64), Rb, coff, w["top_k"])
    assert sorted(ids_h[0].tolist()) == sorted(ids_ref[0].tolist()) == w["planted"].tolist()
    assert sc_ref[0].min() - np.delete(D_ref[0], ids_ref[0]).max() >= 0.05
    mK, m = oracle.gather_rows(Kb, coff, ids_ref[0])
    mV, _ = oracle.gather_rows(Vb, coff, ids_ref[0])
    ref = oracle.sparse_attn(w["Q"].astype(np.float64), mK, mV, [0, m], w["K_loc"].astype(np.float64),
                             w["V_loc"].astype(np.float64), w["top_k"], W.scale_of(w["d"]), w["theta"])
    P.assert_attn_close(O.cpu().numpy(), ref, 1e-3, "tiny fp32 pipeline")
    ctx.close()


@pytest.mark.timeout(400)
def test_qwen_bf16_layer_end_to_end(gpu, msa):
    """2,000 documents with lengths U[128, 1024] (~1.15M tokens), chunk 64,
    32/8 heads, d 128, 256-token routing query, top-16 with 16 planted
    documents, then a 1-token decode over the gathered rows + 257 local."""
    import torch
    from msa_synth import device
    w = W.qwen_bf16_layer()
    Hq, Hkv, d, c, k = w["Hq"], w["Hkv"], w["d"], w["chunk"], w["top_k"]
    ctx = msa.msa_ctx_create(0, d, w["theta"], 16384)
    tok, T = w["tok_off"], w["T"]
    coff, max_len = msa.msa_chunk_offsets(tok, c, with_max_len=True)
    N = int(coff[-1])
    K = torch.empty((T, Hkv, d), dtype=torch.bfloat16, device="cuda")
    V = torch.empty_like(K)
    device.fill_counter_bf16(K, w["seed"], w["K_stream"], 0)
    device.fill_counter_bf16(V, w["seed"], w["V_stream"], 0)
    KVbar = torch.empty((N, 2, Hkv, d), dtype=torch.bfloat16, device="cuda")
    Krbar = torch.empty((N, Hkv, d), dtype=torch.bfloat16, device="cuda")
    msa.msa_encode_pool(ctx, K, V, W.dev_bf16(w["Kr"]), torch.from_numpy(tok).cuda(),
                        torch.from_numpy(coff).cuda(), KVbar, Krbar, c, max_len)
    del K, V
    ids = torch.empty((1, k), dtype=torch.int32, device="cuda")
    ws = msa.workspace(msa.msa_route_workspace_size(1, 1, w["Tq"], Hq, Hkv, N, w["n_docs"], k))
    msa.msa_route(ctx, W.dev_bf16(w["Qr"]), Krbar, torch.from_numpy(coff).cuda(), k, ids, ws)
    ids_h = ids.cpu().numpy()
    O = _gather_and_attend(torch, msa, ctx, KVbar, coff, ids_h, W.dev_bf16(w["Q"]), W.dev_bf16(w["K_loc"]),
                           W.dev_bf16(w["V_loc"]), k, "bf16")
    KVbar_h = W.widen(W.host_bits(KVbar), "bf16")

    # oracle routing on its own pooled, bf16-rounded routing keys
    Rb = np.empty((N, Hkv, d))
    for doc in range(w["n_docs"]):
        s, e = tok[doc], tok[doc + 1]
        Rb[coff[doc]:coff[doc + 1]] = oracle.chunk_mean(W.widen(w["Kr"][s:e], "bf16"), [0, e - s], c)
    Rb = W.round_store(Rb, "bf16")
    ids_ref, sc_ref, _, D_ref = oracle.route(W.widen(w["Qr"], "bf16"), Rb, coff, k)
    assert sorted(ids_h[0].tolist()) == sorted(ids_ref[0].tolist()) == w["planted"].tolist()
    assert sc_ref[0].min() - np.delete(D_ref[0], ids_ref[0]).max() >= 0.05

    # oracle pooling of the selected documents (raw K/V regenerated) and a sample of others
    sample = sorted(set(ids_ref[0].tolist()) | set(np.random.default_rng(9).integers(0, w["n_docs"], 8).tolist()))
    pooled = {}
    for doc in sample:
        s, e = int(tok[doc]), int(tok[doc + 1])
        Kd = W.widen(W.counter_rows(w["seed"], w["K_stream"], s, e, Hkv, d), "bf16")
        Vd = W.widen(W.counter_rows(w["seed"], w["V_stream"], s, e, Hkv, d), "bf16")
        Kb, Vb, _ = oracle.encode_pool(Kd, Vd, Vd, [0, e - s], c, w["theta"])
        pooled[doc] = (Kb, Vb)
        assert W.rel_row_err(KVbar_h[coff[doc]:coff[doc + 1], 0], Kb) <= 2e-2
        assert W.rel_row_err(KVbar_h[coff[doc]:coff[doc + 1], 1], Vb) <= 2e-2
    sel = sorted(ids_ref[0].tolist())
    mK = W.round_store(np.concatenate([pooled[i][0] for i in sel]), "bf16")
    mV = W.round_store(np.concatenate([pooled[i][1] for i in sel]), "bf16")
    ref = oracle.sparse_attn(W.widen(w["Q"], "bf16"), mK, mV, [0, len(mK)], W.widen(w["K_loc"], "bf16"),
                             W.widen(w["V_loc"], "bf16"), k, W.scale_of(d), w["theta"])
    got = W.widen(W.host_bits(O), "bf16")
    P.assert_attn_close(got, ref, 2e-2, "Qwen-shaped layer decode")
    ctx.close()
