"""Parity at the full workload sizes, in the launch configurations bench.py
times (GPU only).  Where the oracle cannot cover every output in seconds, it
checks sampled outputs one by one and the properties that hold at any size
(planted documents recovered with their margin).  Tolerances as in
test_gpu_parity.py."""

import math

import numpy as np
import pytest

import msa_synth
import oracle
from tests import peaked as P
from tests import workloads as W

pytestmark = pytest.mark.gpu

Hq, Hkv, D, C = 32, 8, 128, 64
MFMA_TOL = 3e-3     # batched decode on the matrix cores: U rounded to bf16, |delta s| <= 2^-9
GEMM_TOL = 5e-3     # prefill GEMM: U and the unit keys rounded to bf16, |delta s| <= 2^-8
VALU_TOL = 1e-4


@pytest.fixture(scope="module")
def env(gpu):
    import torch
    import long_context_memory_chunk_amd as msa
    from msa_synth import device
    msa.lib()
    ctx = msa.msa_ctx_create(0, D, 1e6, 16384)
    yield torch, msa, device, ctx
    ctx.close()


def _pinned_layer(torch, device, seed, layer, N):
    host = torch.empty((N, 2, Hkv, D), dtype=torch.bfloat16, pin_memory=True)
    device.fill_counter_bf16((host.data_ptr(), host.numel()), seed, W.kvbar_stream(layer), 0)
    torch.cuda.synchronize()
    return host


def _oracle_scores_blocked(Qr64, seed, layer, coff, planted_rows, block=200_000):
    """Oracle chunk scores over a whole counter-generated layer, block by block,
    with the planted rows written in (regenerated on the host)."""
    N = int(coff[-1])
    out = np.empty((Qr64.shape[0], N))
    for a in range(0, N, block):
        e = min(a + block, N)
        kb = W.counter_bf16_threads(seed, W.krbar_stream(layer), a * Hkv * D, (e - a) * Hkv * D).reshape(-1, Hkv, D)
        for (r0, r1), rows in planted_rows:
            lo, hi = max(r0, a), min(r1, e)
            if lo < hi:
                kb[lo - a:hi - a] = rows[lo - r0:hi - r0]
        out[:, a:e] = oracle.chunk_scores(Qr64, W.widen(kb, "bf16"))
    return out


@pytest.mark.timeout(900)
def test_decode_100m_layer_full_oracle_topk(env):
    """The 100M-token bank's layer 0 (1,562,500 chunk rows, ~200K documents):
    the decode scan's chunk scores and top-16 against the oracle over every
    chunk; then gather from the pinned host store and attention."""
    torch, msa, device, ctx = env
    seed, k = 0, 16
    lens = msa_synth.lognormal_lengths(seed, 100_000_000)
    coff = msa_synth.ceil_chunk_offsets(lens, C)
    n_docs, N = len(lens), int(coff[-1])
    assert N == 1_562_500
    Kr = torch.empty((N, Hkv, D), dtype=torch.bfloat16, device="cuda")
    device.fill_counter_bf16(Kr, seed, W.krbar_stream(0), 0)
    planted = msa_synth.pick_planted(seed, 50, n_docs, k)
    Qr_h = msa_synth.normal_bf16(seed, 100, (1, 1, Hq, D))
    q = msa_synth.bf16_bits_to_f32(Qr_h)[0, 0]
    prow = []
    for j, d in enumerate(planted):
        rows = W.planted_pooled(seed, 0, q, Hkv, int(coff[d + 1] - coff[d]), tag=j)
        Kr[coff[d]:coff[d + 1]].copy_(W.dev_bf16(rows))
        prow.append(((int(coff[d]), int(coff[d + 1])), rows))
    ids = torch.empty((1, k), dtype=torch.int32, device="cuda")
    ch = torch.empty((1, N), dtype=torch.float32, device="cuda")
    dc = torch.empty((1, n_docs), dtype=torch.float32, device="cuda")
    sc = torch.empty((1, k), dtype=torch.float32, device="cuda")
    ws = msa.workspace(msa.msa_route_workspace_size(1, 1, 1, Hq, Hkv, N, n_docs, k))
    msa.msa_route(ctx, W.dev_bf16(Qr_h), Kr, torch.from_numpy(coff).cuda(), k, ids, ws, out_scores=sc,
                  out_chunk=ch, out_doc=dc)
    torch.cuda.synchronize()
    del Kr
    c_ref = _oracle_scores_blocked(W.widen(Qr_h, "bf16"), seed, 0, coff, prow)
    D_ref = oracle.doc_scores(c_ref, coff)
    ids_ref, sc_ref = oracle.topk_docs(D_ref, k)
    got = ids.cpu().numpy()
    assert sorted(got[0].tolist()) == sorted(ids_ref[0].tolist()) == planted.tolist()
    assert sc_ref[0].min() - np.delete(D_ref[0], ids_ref[0]).max() >= 0.05
    assert np.max(np.abs(ch.cpu().numpy() - c_ref)) <= VALU_TOL
    assert np.max(np.abs(dc.cpu().numpy() - D_ref)) <= VALU_TOL

    # gather (hipMemcpyAsync from the pinned store) and decode attention, 2,048 local tokens
    host = _pinned_layer(torch, device, seed, 0, N)
    cap = int(np.sort(np.diff(coff))[-k:].sum())            # rows of the k largest documents
    dst = torch.empty((cap, 2, Hkv, D), dtype=torch.bfloat16, device="cuda")
    mo_h = torch.zeros(2, dtype=torch.int64, pin_memory=True)
    mo_d = torch.zeros(2, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    msa.msa_gather(host, 2 * Hkv * D * 2, N, coff, got.astype(np.int32), k, dst, cap, mo_h, mo_d, side=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    full, dst = dst, dst[:int(mo_h[1])]
    L = 2048
    Qh = msa_synth.normal_bf16(seed, 200, (1, 1, Hq, D))
    Klh = msa_synth.normal_bf16(seed, 300, (1, L, Hkv, D))
    Vlh = msa_synth.normal_bf16(seed, 400, (1, L, Hkv, D))
    O = torch.empty((1, 1, Hq, D), dtype=torch.bfloat16, device="cuda")
    wsa = msa.workspace(msa.msa_sparse_attn_workspace_size(1, 1, 1, Hq, Hkv, cap, L))
    msa.msa_sparse_attn(ctx, W.dev_bf16(Qh), full, mo_d, cap, W.dev_bf16(Klh), W.dev_bf16(Vlh), k,
                        1 / math.sqrt(D), O, wsa)
    torch.cuda.synchronize()
    sel = sorted(int(d) for d in ids_ref[0])
    rows = np.concatenate([msa_synth.counter_bf16(seed, W.kvbar_stream(0), int(coff[d]) * 2 * Hkv * D,
                                                  int(coff[d + 1] - coff[d]) * 2 * Hkv * D).reshape(-1, 2, Hkv, D)
                           for d in sel])
    assert np.array_equal(W.host_bits(dst), rows)                    # byte-exact gather
    kv = W.widen(rows, "bf16")
    ref = oracle.sparse_attn(W.widen(Qh, "bf16"), kv[:, 0], kv[:, 1], [0, len(kv)], W.widen(Klh, "bf16"),
                             W.widen(Vlh, "bf16"), k, 1 / math.sqrt(D), 1e6)
    P.assert_attn_close(W.widen(W.host_bits(O), "bf16"), ref, 2e-2, "100M layer decode")

    # the same layer through msa_gather_attn, as the routed decode step runs it
    # (a 2,048-row capacity: most copy workgroups past the gathered rows)
    dst2 = torch.full((cap, 2, Hkv, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    mo2 = torch.full((2,), -7, dtype=torch.int64, device="cuda")
    O2 = torch.full((1, 1, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    ids_dev = torch.from_numpy(got.astype(np.int32)).cuda()
    wsga = msa.workspace(msa.msa_gather_attn_workspace_size(1, 1, 1, Hq, Hkv, k, cap, cap, L))
    msa.msa_gather_attn(ctx, host, 2 * Hkv * D * 2, N, torch.from_numpy(coff).cuda(), ids_dev, dst2, cap, mo2,
                        W.dev_bf16(Qh), cap, W.dev_bf16(Klh), W.dev_bf16(Vlh), k, 1 / math.sqrt(D), O2, wsga)
    torch.cuda.synchronize()
    assert mo2.cpu().tolist() == [0, len(rows)]
    assert np.array_equal(W.host_bits(dst2[:len(rows)]), rows)
    P.assert_attn_close(W.widen(W.host_bits(O2), "bf16"), ref, 2e-2, "100M layer decode, one call")


@pytest.mark.timeout(900)
def test_chunk_level_topk_100m_layer(env):
    """Chunk-level selection (documents of one chunk each: offsets 0, 1, ..., N)
    on the 100M-token bank's layer 0: the top-16 chunks against the oracle over
    every chunk, then both gathers copy one row per selected chunk."""
    torch, msa, device, ctx = env
    seed, k = 0, 16
    lens = msa_synth.lognormal_lengths(seed, 100_000_000)
    N = int(msa_synth.ceil_chunk_offsets(lens, C)[-1])
    coff = np.arange(N + 1, dtype=np.int64)
    Kr = torch.empty((N, Hkv, D), dtype=torch.bfloat16, device="cuda")
    device.fill_counter_bf16(Kr, seed, W.krbar_stream(0), 0)
    planted = msa_synth.pick_planted(seed, 60, N, k)
    Qr_h = msa_synth.normal_bf16(seed, 101, (1, 1, Hq, D))
    q = msa_synth.bf16_bits_to_f32(Qr_h)[0, 0]
    prow = []
    for j, r in enumerate(planted):
        rows = W.planted_pooled(seed, 0, q, Hkv, 1, tag=500 + j)
        Kr[int(r):int(r) + 1].copy_(W.dev_bf16(rows))
        prow.append(((int(r), int(r) + 1), rows))
    coff_d = torch.from_numpy(coff).cuda()
    ids = torch.empty((1, k), dtype=torch.int32, device="cuda")
    sc = torch.empty((1, k), dtype=torch.float32, device="cuda")
    ws = msa.workspace(msa.msa_route_workspace_size(1, 1, 1, Hq, Hkv, N, N, k))
    msa.msa_route(ctx, W.dev_bf16(Qr_h), Kr, coff_d, k, ids, ws, out_scores=sc)
    torch.cuda.synchronize()
    del Kr
    c_ref = _oracle_scores_blocked(W.widen(Qr_h, "bf16"), seed, 0, coff, prow)
    ids_ref, sc_ref = oracle.topk_docs(c_ref, k)             # documents of one chunk: chunk scores
    got = ids.cpu().numpy()
    assert sorted(got[0].tolist()) == sorted(ids_ref[0].tolist()) == sorted(planted.tolist())
    assert sc_ref[0].min() - np.delete(c_ref[0], ids_ref[0]).max() >= 0.05
    assert np.max(np.abs(sc.cpu().numpy() - sc_ref)) <= VALU_TOL

    # both gathers: one 4 KB row per selected chunk, in ascending chunk order
    host = _pinned_layer(torch, device, seed, 0, N)
    dst = torch.empty((k, 2, Hkv, D), dtype=torch.bfloat16, device="cuda")
    mo_h = torch.zeros(2, dtype=torch.int64, pin_memory=True)
    mo_d = torch.zeros(2, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    msa.msa_gather(host, 2 * Hkv * D * 2, N, coff, got.astype(np.int32), k, dst, k, mo_h, mo_d, side=side)
    torch.cuda.current_stream().wait_stream(side)
    dst2 = torch.empty_like(dst)
    mo2 = torch.zeros(2, dtype=torch.int64, device="cuda")
    wsg = msa.workspace(msa.msa_gather_device_workspace_size(1, k, k))
    msa.msa_gather_device(ctx, host, 2 * Hkv * D * 2, N, coff_d, ids, dst2, k, mo2, wsg)
    torch.cuda.synchronize()
    rows = np.concatenate([msa_synth.counter_bf16(seed, W.kvbar_stream(0), int(r) * 2 * Hkv * D, 2 * Hkv * D)
                           .reshape(1, 2, Hkv, D) for r in sorted(int(x) for x in ids_ref[0])])
    assert int(mo_h[1]) == k and mo2.cpu().tolist() == [0, k]
    assert np.array_equal(W.host_bits(dst), rows)
    assert np.array_equal(W.host_bits(dst2), rows)


@pytest.mark.timeout(900)
def test_batch32_10m_layer_full_oracle(env):
    """32 single-token queries against one layer of the 10M-token bank
    (156,250 chunk rows, ~20K documents), matrix-core routing: every query's
    top-16 against the oracle over every chunk; device gather; attention,
    both as two calls and as msa_gather_attn."""
    torch, msa, device, ctx = env
    seed, k, B, L = 0, 16, 32, 2048
    lens = msa_synth.lognormal_lengths(seed, 10_000_000)
    coff = msa_synth.ceil_chunk_offsets(lens, C)
    n_docs, N = len(lens), int(coff[-1])
    assert N == 156_250
    Kr = torch.empty((N, Hkv, D), dtype=torch.bfloat16, device="cuda")
    device.fill_counter_bf16(Kr, seed, W.krbar_stream(0), 0)
    Qr_h = msa_synth.normal_bf16(seed, 800, (B, 1, Hq, D))
    qf = msa_synth.bf16_bits_to_f32(Qr_h)
    planted = [msa_synth.pick_planted(seed + 100 + b, 50, n_docs, k) for b in range(B)]
    taken, prow = set(), []
    for b in range(B):      # disjoint planted sets per query, as the batched decode workload draws them
        if set(planted[b].tolist()) & taken:
            planted[b] = msa_synth.pick_planted(seed + 100 + b, 50, n_docs, k, exclude=taken)
        taken |= set(planted[b].tolist())
    for b in range(B):
        for j, d in enumerate(planted[b]):
            rows = W.planted_pooled(seed, 0, qf[b, 0], Hkv, int(coff[d + 1] - coff[d]), tag=1000 + b * k + j)
            Kr[coff[d]:coff[d + 1]].copy_(W.dev_bf16(rows))
            prow.append(((int(coff[d]), int(coff[d + 1])), rows))
    ids = torch.empty((B, k), dtype=torch.int32, device="cuda")
    ch = torch.empty((B, N), dtype=torch.float32, device="cuda")
    ws = msa.workspace(msa.msa_route_workspace_size(1, B, 1, Hq, Hkv, N, n_docs, k))
    coff_dev = torch.from_numpy(coff).cuda()
    msa.msa_route(ctx, W.dev_bf16(Qr_h), Kr, coff_dev, k, ids, ws, out_chunk=ch)
    torch.cuda.synchronize()
    c_ref = _oracle_scores_blocked(W.widen(Qr_h, "bf16"), seed, 0, coff, prow)
    D_ref = oracle.doc_scores(c_ref, coff)
    ids_ref, sc_ref = oracle.topk_docs(D_ref, k)
    got = ids.cpu().numpy()
    for b in range(B):
        assert sorted(got[b].tolist()) == sorted(ids_ref[b].tolist()) == planted[b].tolist()
        assert sc_ref[b].min() - np.delete(D_ref[b], ids_ref[b]).max() >= 0.05
    assert np.max(np.abs(ch.cpu().numpy() - c_ref)) <= MFMA_TOL

    host = _pinned_layer(torch, device, seed, 0, N)
    max_rows = int(np.sort(np.diff(coff))[-k:].sum())
    cap = B * max_rows
    dst = torch.empty((cap, 2, Hkv, D), dtype=torch.bfloat16, device="cuda")
    mo = torch.zeros(B + 1, dtype=torch.int64, device="cuda")
    wsg = msa.workspace(msa.msa_gather_device_workspace_size(B, k, cap))
    msa.msa_gather_device(ctx, host, 2 * Hkv * D * 2, N, coff_dev, ids, dst, cap, mo, wsg)
    Qh = msa_synth.normal_bf16(seed, 900, (B, 1, Hq, D))
    Kl = torch.empty((B, L, Hkv, D), dtype=torch.bfloat16, device="cuda")
    Vl = torch.empty_like(Kl)
    device.fill_counter_bf16(Kl, seed, 1200, 0)
    device.fill_counter_bf16(Vl, seed, 1300, 0)
    O = torch.empty((B, 1, Hq, D), dtype=torch.bfloat16, device="cuda")
    wsa = msa.workspace(msa.msa_sparse_attn_workspace_size(1, B, 1, Hq, Hkv, max_rows, L))
    msa.msa_sparse_attn(ctx, W.dev_bf16(Qh), dst, mo, max_rows, Kl, Vl, k, 1 / math.sqrt(D), O, wsa)
    torch.cuda.synchronize()
    mo_np = mo.cpu().numpy()
    got_o = W.widen(W.host_bits(O), "bf16")
    refs = {}
    for b in (0, 7, 31):
        sel = sorted(int(d) for d in ids_ref[b])
        rows = np.concatenate([msa_synth.counter_bf16(seed, W.kvbar_stream(0), int(coff[d]) * 2 * Hkv * D,
                                                      int(coff[d + 1] - coff[d]) * 2 * Hkv * D).reshape(-1, 2, Hkv, D)
                               for d in sel])
        assert np.array_equal(W.host_bits(dst[mo_np[b]:mo_np[b + 1]]), rows)
        kv = W.widen(rows, "bf16")
        klb = W.widen(W.counter_rows(seed, 1200, b * L, (b + 1) * L, Hkv, D), "bf16")
        vlb = W.widen(W.counter_rows(seed, 1300, b * L, (b + 1) * L, Hkv, D), "bf16")
        ref = oracle.sparse_attn(W.widen(Qh[b:b + 1], "bf16"), kv[:, 0], kv[:, 1], [0, len(kv)], klb[None],
                                 vlb[None], k, 1 / math.sqrt(D), 1e6)
        P.assert_attn_close(got_o[b], ref[0], 2e-2, f"batch32 query {b}")
        refs[b] = ref[0]

    # the same layer through msa_gather_attn, as the batched decode step runs
    # it (the copy beside the local keys' attention): the same rows and
    # offsets, the same attention within rounding, and the oracle's bar
    dst2 = torch.empty_like(dst)
    mo2 = torch.zeros_like(mo)
    O2 = torch.empty_like(O)
    wsga = msa.workspace(msa.msa_gather_attn_workspace_size(1, B, 1, Hq, Hkv, k, cap, max_rows, L))
    msa.msa_gather_attn(ctx, host, 2 * Hkv * D * 2, N, coff_dev, ids, dst2, cap, mo2, W.dev_bf16(Qh), max_rows,
                        Kl, Vl, k, 1 / math.sqrt(D), O2, wsga)
    torch.cuda.synchronize()
    assert np.array_equal(mo2.cpu().numpy(), mo_np)
    assert np.array_equal(W.host_bits(dst2[:mo_np[B]]), W.host_bits(dst[:mo_np[B]]))
    got_o2 = W.widen(W.host_bits(O2), "bf16")
    for b, ref in refs.items():
        P.assert_attn_close(got_o2[b], ref, 2e-2, f"batch32 query {b}, one call")
    assert float(np.max(np.abs(got_o2 - got_o))) <= 1e-2


@pytest.mark.timeout(900)
def test_prefill8k_10m_layer_sampled(env):
    """An 8,192-token query against one layer of the 10M-token bank on the
    matrix cores (2.62 TFLOP folded), top-32 with 32 planted documents; then
    causal prefill over [gathered rows ; 8,192 local].  The oracle checks the
    chunk scores of every planted chunk and 3,000 random chunks over all 8,192
    tokens, planted recovery, and the attention output of sampled tokens."""
    torch, msa, device, ctx = env
    seed, k, T = 0, 32, 8192
    lens = msa_synth.lognormal_lengths(seed, 10_000_000)
    coff = msa_synth.ceil_chunk_offsets(lens, C)
    n_docs, N = len(lens), int(coff[-1])
    Kr = torch.empty((N, Hkv, D), dtype=torch.bfloat16, device="cuda")
    device.fill_counter_bf16(Kr, seed, W.krbar_stream(0), 0)
    Qr_h = msa_synth.normal_bf16(seed, 700, (1, T, Hq, D))
    planted = msa_synth.pick_planted(seed, 51, n_docs, k)
    toks = np.random.default_rng(seed + 52).integers(0, T, size=k)
    qf = msa_synth.bf16_bits_to_f32(Qr_h)
    prow = {}
    for j, d in enumerate(planted):
        rows = W.planted_pooled(seed, 0, qf[0, toks[j]], Hkv, int(coff[d + 1] - coff[d]), tag=j)
        Kr[coff[d]:coff[d + 1]].copy_(W.dev_bf16(rows))
        prow[int(d)] = rows
    ids = torch.empty((1, k), dtype=torch.int32, device="cuda")
    ch = torch.empty((1, N), dtype=torch.float32, device="cuda")
    coff_dev = torch.from_numpy(coff).cuda()
    ws = msa.workspace(msa.msa_route_workspace_size(1, 1, T, Hq, Hkv, N, n_docs, k))
    msa.msa_route(ctx, W.dev_bf16(Qr_h), Kr, coff_dev, k, ids, ws, out_chunk=ch)
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    assert sorted(got[0].tolist()) == planted.tolist()
    chn = ch.cpu().numpy()[0]
    # sampled chunks: all chunks of the planted documents + 3,000 random chunks
    rng = np.random.default_rng(5)
    samp = sorted(set(rng.integers(0, N, 3000).tolist()))
    Qr64 = W.widen(Qr_h, "bf16")
    kb = np.stack([W.counter_rows(seed, W.krbar_stream(0), n, n + 1, Hkv, D)[0] for n in samp])
    pd = set(int(d) for d in planted)
    for i, n in enumerate(samp):                    # a sampled chunk may belong to a planted document
        dd = int(np.searchsorted(coff, n, side="right")) - 1
        if dd in pd:
            kb[i] = prow[dd][n - coff[dd]]
    c_s = oracle.chunk_scores(Qr64, W.widen(kb, "bf16"))[0]
    assert np.max(np.abs(chn[samp] - c_s)) <= GEMM_TOL
    p_idx = np.concatenate([np.arange(coff[d], coff[d + 1]) for d in planted])
    p_rows = np.concatenate([prow[int(d)] for d in planted])
    c_p = oracle.chunk_scores(Qr64, W.widen(p_rows, "bf16"))[0]
    assert np.max(np.abs(chn[p_idx] - c_p)) <= GEMM_TOL
    # the planted documents beat every sampled chunk by the margin
    D_p = oracle.doc_scores(c_p[None], np.concatenate([[0], np.cumsum(np.diff(coff)[planted])]))[0]
    assert D_p.min() - c_s[[i for i, n in enumerate(samp) if int(np.searchsorted(coff, n, side='right')) - 1 not in pd]].max() >= 0.05

    # gather + causal prefill attention, sampled tokens against the oracle
    host = _pinned_layer(torch, device, seed, 0, N)
    cap = int(np.sort(np.diff(coff))[-k:].sum())            # rows of the k largest documents
    dst = torch.empty((cap, 2, Hkv, D), dtype=torch.bfloat16, device="cuda")
    mo_h = torch.zeros(2, dtype=torch.int64, pin_memory=True)
    mo_d = torch.zeros(2, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    msa.msa_gather(host, 2 * Hkv * D * 2, N, coff, got.astype(np.int32), k, dst, cap, mo_h, mo_d, side=side)
    torch.cuda.current_stream().wait_stream(side)
    Q = torch.empty((1, T, Hq, D), dtype=torch.bfloat16, device="cuda")
    Kl = torch.empty((1, T, Hkv, D), dtype=torch.bfloat16, device="cuda")
    Vl = torch.empty_like(Kl)
    for t_, st in ((Q, 710), (Kl, 711), (Vl, 712)):
        device.fill_counter_bf16(t_, seed, st, 0)
    O = torch.empty_like(Q)
    wsa = msa.workspace(msa.msa_sparse_attn_workspace_size(1, 1, T, Hq, Hkv, cap, T))
    msa.msa_sparse_attn(ctx, Q, dst, mo_d, cap, Kl, Vl, k, 1 / math.sqrt(D), O, wsa)
    torch.cuda.synchronize()
    rows = W.widen(np.concatenate([msa_synth.counter_bf16(seed, W.kvbar_stream(0), int(coff[d]) * 2 * Hkv * D,
                                                          int(coff[d + 1] - coff[d]) * 2 * Hkv * D).reshape(-1, 2, Hkv, D)
                                   for d in sorted(int(x) for x in planted)]), "bf16")
    got_o = W.host_bits(O)
    for i in (0, 1, 127, 128, 4095, 8191):
        qi = W.widen(msa_synth.counter_bf16(seed, 710, i * Hq * D, Hq * D).reshape(1, 1, Hq, D), "bf16")
        kl = W.widen(W.counter_rows(seed, 711, 0, i + 1, Hkv, D), "bf16")
        vl = W.widen(W.counter_rows(seed, 712, 0, i + 1, Hkv, D), "bf16")
        ref = oracle.sparse_attn(qi, rows[:, 0], rows[:, 1], [0, len(rows)], kl[None], vl[None], k,
                                 1 / math.sqrt(D), 1e6)
        P.assert_attn_close(W.widen(got_o[0, i], "bf16"), ref[0, 0], 2e-2, f"8K prefill token {i}")


@pytest.mark.timeout(900)
def test_encode_10m_layer_sampled(env):
    """The offline encode of one layer of the 10M-token bank (raw K, V, Kr
    [10M, 8, 128] bf16, log-normal lengths up to 8,192 tokens), launched as
    bench.py's encode workload launches it; the oracle pools 60 documents
    (the longest, the shortest, the first, the last and 56 drawn at random)
    from their regenerated raw rows."""
    torch, msa, device, ctx = env
    import bench
    seed = 0
    lens, tok, (K, V, Kr) = bench.encode_10m_inputs(seed, torch, msa_synth, device)
    coff, max_len = msa.msa_chunk_offsets(tok, C, with_max_len=True)
    N = int(coff[-1])
    KVbar = torch.full((N, 2, Hkv, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    Krbar = torch.full((N, Hkv, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    msa.msa_encode_pool(ctx, K, V, Kr, torch.from_numpy(tok).cuda(), torch.from_numpy(coff).cuda(),
                        KVbar, Krbar, C, max_len)
    torch.cuda.synchronize()
    del K, V, Kr
    assert bool(torch.isfinite(KVbar).all()) and bool(torch.isfinite(Krbar).all())
    n_docs = len(lens)
    docs = {int(np.argmax(lens)), int(np.argmin(lens)), 0, n_docs - 1}
    docs |= set(np.random.default_rng(9).choice(n_docs, 56, replace=False).tolist())
    for d in sorted(docs):
        s, e, c0, c1 = int(tok[d]), int(tok[d + 1]), int(coff[d]), int(coff[d + 1])
        raw = [W.widen(W.counter_rows(seed, st, s, e, Hkv, D), "bf16") for st in bench.ENCODE_STREAMS]
        Kb, Vb, Rb = oracle.encode_pool(*raw, np.array([0, e - s]), C, 1e6)
        kv = W.widen(W.host_bits(KVbar[c0:c1]), "bf16")
        kr = W.widen(W.host_bits(Krbar[c0:c1]), "bf16")
        for got, ref in ((kv[:, 0], Kb), (kv[:, 1], Vb), (kr, Rb)):
            assert W.rel_row_err(got, ref) <= 2 ** -8 + 1e-5, d
