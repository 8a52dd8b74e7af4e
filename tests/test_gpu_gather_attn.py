"""msa_gather_attn (the device gather and the attention in one call) against
the oracle, through the C ABI (GPU only).

Each query's memory rows are the peaked inputs of tests/peaked.py, cut into
top_k documents (some empty) that sit at ascending ids among distractor
documents of a pinned host bank; the ids are given shuffled.  The gather must
lay the selected documents out in ascending id order (neo-ai.one MSA article,
推論パイプライン, Fig. 3: only the selected K̄/V̄ are loaded), which
reproduces the planted rows exactly, so the call is checked three ways:
the gathered bytes and mem_off against oracle.gather_rows, O against the
oracle's attention over those rows at the peaked bar (max|O - O_ref| <= 2e-2
and <= 2e-2 max|O_ref|; 1e-3 in fp32), and O against msa_gather_device
followed by msa_sparse_attn on the same inputs (the same softmax, its
partials merged in another order).
"""

import numpy as np
import pytest

import msa_synth
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


def _bank(w, k, seed):
    """Host bank (bf16 bits [N, 2, Hkv, d]), document offsets and shuffled ids
    [B, k] whose ascending-id gather gives each query's rows of w["KV"]."""
    rng = np.random.default_rng(seed)
    mem_off = np.asarray(w["mem_off"], dtype=np.int64)
    B = len(mem_off) - 1
    Hkv = w["Kl"].shape[2]
    docs, ids = [], []
    for b in range(B):
        for t in range(int(rng.integers(1, 4))):                       # distractors before the query's documents
            docs.append(msa_synth.normal_bf16(seed, 100 + 10 * b + t, (int(rng.integers(1, 9)), 2, Hkv, D)))
        a, e = int(mem_off[b]), int(mem_off[b + 1])
        cuts = np.sort(rng.integers(a, e + 1, size=k - 1)) if k > 1 else np.zeros(0, dtype=np.int64)
        edges = [a, *cuts.tolist(), e]
        mine = []
        for j in range(k):
            mine.append(len(docs))
            docs.append(w["KV"][edges[j]:edges[j + 1]])
        ids.append(rng.permutation(np.array(mine, dtype=np.int32)))
    docs.append(msa_synth.normal_bf16(seed, 99, (3, 2, Hkv, D)))          # one after the last query's
    coff = msa_synth.prefix_offsets([len(x) for x in docs])
    return np.concatenate(docs), coff, np.stack(ids)


def _run(torch, msa, ctx, w, k, seed, dtype="bf16", cap_extra=0, fused=True):
    bank, coff, ids = _bank(w, k, seed)
    B, Tq, Hq, _ = w["Q"].shape
    L, Hkv = w["Kl"].shape[1], w["Kl"].shape[2]
    rows = np.diff(w["mem_off"])
    max_rows = int(rows.max()) if len(rows) else 0
    cap = int(rows.sum()) + cap_extra
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    esz = 2 if dtype == "bf16" else 4

    def put(bits):
        return W.dev_bf16(bits) if dtype == "bf16" else W.dev_f32(oracle.bf16_bits_to_f64(bits))

    host = torch.empty(bank.shape, dtype=tdt, pin_memory=True)
    host.copy_(put(bank).cpu())
    N = bank.shape[0]
    coff_dev = torch.from_numpy(coff).cuda()
    ids_dev = torch.from_numpy(ids).cuda()
    Q, Kl, Vl = put(w["Q"]), put(w["Kl"]), put(w["Vl"])
    row_bytes = 2 * Hkv * D * esz
    dst = torch.full((max(cap, 1), 2, Hkv, D), float("nan"), dtype=tdt, device="cuda")
    mo = torch.full((B + 1,), -7, dtype=torch.int64, device="cuda")
    O = torch.full((B, Tq, Hq, D), float("nan"), dtype=tdt, device="cuda")
    dt = 1 if dtype == "bf16" else 0
    if fused:
        ws = msa.workspace(msa.msa_gather_attn_workspace_size(dt, B, Tq, Hq, Hkv, k, cap, max_rows, L))
        print(f"[gather_attn] B={B} Tq={Tq} G={Hq // Hkv} L={L} rows={rows.tolist()[:8]} k={k} cap={cap} {dtype}",
              flush=True)
        msa.msa_gather_attn(ctx, host, row_bytes, N, coff_dev, ids_dev, dst, cap, mo, Q, max_rows, Kl, Vl,
                            w["qoff"], w["scale"], O, ws)
    else:
        wsg = msa.workspace(msa.msa_gather_device_workspace_size(B, k, cap))
        msa.msa_gather_device(ctx, host, row_bytes, N, coff_dev, ids_dev, dst, cap, mo, wsg)
        wsa = msa.workspace(msa.msa_sparse_attn_workspace_size(dt, B, Tq, Hq, Hkv, max_rows, L))
        msa.msa_sparse_attn(ctx, Q, dst, mo, max_rows, Kl, Vl, w["qoff"], w["scale"], O, wsa)
    torch.cuda.synchronize()
    return bank, coff, ids, W.widen(W.host_bits(dst), dtype), mo.cpu().numpy(), W.widen(W.host_bits(O), dtype)


# (seed, B, Tq, Hq, Hkv, L, memory rows per query, top_k)
CASES = [
    (61, 1, 1, 32, 8, 2048, [125], 16),                 # the one-query copy beside the local keys
    (62, 4, 1, 32, 8, 700, [100, 0, 37, 260], 8),       # the plan + bounded copy; a query with no memory rows
    (63, 3, 4, 16, 16, 300, [50, 130, 9], 5),           # G = 1, four query tokens per row
    (64, 2, 1, 16, 2, 257, [300, 1], 3),                # G = 8, a ragged local tail
    (65, 2, 2, 8, 4, 128, [64, 65], 4),                 # G = 2
    (66, 8, 1, 32, 8, 2048, [60, 200, 130, 90, 1, 170, 150, 77], 16),
    (70, 1, 63, 32, 8, 300, [90], 6),                  # Tq = 63: the largest query block on the fused path
    (71, 1, 64, 32, 8, 256, [100], 8),                 # Tq = 64: the prefill kernel, after the gather
    (72, 2, 3, 32, 2, 200, [30, 70], 5),               # G = 16: the split kernel, after the gather
]


@pytest.mark.parametrize("seed,B,Tq,Hq,Hkv,L,rows,k", CASES)
def test_gather_attn_matches_oracle(env, seed, B, Tq, Hq, Hkv, L, rows, k):
    torch, msa, ctx = env
    w = P.peaked_inputs(seed, B, Tq, Hq, Hkv, D, L, rows, k, P.THETA, tokens=list(range(Tq)))
    bank, coff, ids, got_rows, mo, got = _run(torch, msa, ctx, w, k, seed)
    want_off = np.asarray(w["mem_off"], dtype=np.int64)
    assert np.array_equal(mo, want_off)
    for b in range(B):
        ref_rows, m = oracle.gather_rows(bank, coff, ids[b])
        assert m == want_off[b + 1] - want_off[b]
        assert np.array_equal(oracle.f64_to_bf16_bits(got_rows[mo[b]:mo[b + 1]]), ref_rows)
    ref = P.oracle_out(w)
    assert np.max(np.abs(ref)) > 0.25
    P.assert_attn_close(got, ref, 2e-2, f"gather_attn B={B} Tq={Tq} G={Hq // Hkv} L={L}")
    # the same call made as two (gather, then attention): the same softmax
    _, _, _, rows2, mo2, got2 = _run(torch, msa, ctx, w, k, seed, fused=False)
    assert np.array_equal(mo2, mo)
    assert np.array_equal(rows2[:mo[B]], got_rows[:mo[B]])
    diff = float(np.max(np.abs(got - got2)))
    print(f"[gather_attn] max|O - O_two_calls| = {diff:.3e}", flush=True)
    assert diff <= 1e-2 * max(1.0, float(np.max(np.abs(ref))))


def _random_cases(n, seed):
    """Seeded shapes over both copies (one query; the plan and bounded copy
    for B > 1): 1-40 queries of 1-3 tokens, group sizes 1-8 over 1-8 KV
    heads, local contexts of up to 1,500 keys, 0-300 memory rows per query in
    1-16 documents."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = 1 if i % 3 == 0 else int(rng.integers(2, 41))
        Tq = int(rng.integers(1, 4))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 8]))
        L = int(rng.integers(Tq, 1501))
        rows = [int(r) if rng.random() > 0.15 else 0 for r in rng.integers(1, 301, size=B)]
        if B == 1 and rows[0] == 0:
            rows[0] = 1
        cases.append((900 + i, B, Tq, G * Hkv, Hkv, L, rows, int(rng.integers(1, 17))))
    return cases


@pytest.mark.parametrize("seed,B,Tq,Hq,Hkv,L,rows,k", _random_cases(9, 77))
def test_gather_attn_random_shapes(env, seed, B, Tq, Hq, Hkv, L, rows, k):
    torch, msa, ctx = env
    w = P.peaked_inputs(seed, B, Tq, Hq, Hkv, D, L, rows, k, P.THETA, tokens=list(range(Tq)))
    bank, coff, ids, got_rows, mo, got = _run(torch, msa, ctx, w, k, seed)
    want_off = np.asarray(w["mem_off"], dtype=np.int64)
    assert np.array_equal(mo, want_off)
    for b in range(B):
        ref_rows, _ = oracle.gather_rows(bank, coff, ids[b])
        assert np.array_equal(oracle.f64_to_bf16_bits(got_rows[mo[b]:mo[b + 1]]), ref_rows)
    P.assert_attn_close(got, P.oracle_out(w), 2e-2, f"gather_attn random B={B} Tq={Tq} G={Hq // Hkv} L={L}")


@pytest.mark.parametrize("seed,Hq,Hkv,rows,k,cap_extra", [
    (930, 32, 8, [1], 1, 0),        # one memory row
    (931, 32, 8, [8], 2, 0),        # exactly one copy workgroup's rows
    (932, 32, 8, [9], 3, 0),        # a second workgroup with one row
    (933, 8, 8, [61], 5, 0),        # G = 1
    (934, 8, 1, [77], 4, 0),        # one KV head, G = 8 (a 32-unit row)
    (935, 16, 4, [50], 6, 37),      # spare capacity: workgroups with no rows
    (938, 32, 8, [100], 16, 3972),  # 4 rows per copy workgroup: 1,018 + 6 local partials, the most that fit
    (939, 32, 8, [100], 16, 3976),  # past it: 8 rows per copy workgroup (510 + 6 partials)
    (936, 32, 8, [100], 16, 8040),  # 8 rows per workgroup: 1,018 copy workgroups + 6 local partials
    (937, 32, 8, [100], 16, 8080),  # past it: the copy alone, then a launch over the rows
])
def test_gather_attn_one_token_memory_rows_in_the_copy(env, seed, Hq, Hkv, rows, k, cap_extra):
    """A one-token query: the workgroups that copy the memory rows also form
    their attention partials (4 rows per workgroup, or 8 where 4 would give
    more partials than the merge takes), unless even 8 would."""
    torch, msa, ctx = env
    L = 700
    w = P.peaked_inputs(seed, 1, 1, Hq, Hkv, D, L, rows, k, P.THETA)
    bank, coff, ids, got_rows, mo, got = _run(torch, msa, ctx, w, k, seed, cap_extra=cap_extra)
    assert np.array_equal(mo, np.asarray(w["mem_off"], dtype=np.int64))
    ref_rows, _ = oracle.gather_rows(bank, coff, ids[0])
    assert np.array_equal(oracle.f64_to_bf16_bits(got_rows[:mo[1]]), ref_rows)
    ref = P.oracle_out(w)
    P.assert_attn_close(got, ref, 2e-2, f"gather_attn one token G={Hq // Hkv} rows={rows} cap+{cap_extra}")
    _, _, _, _, _, got2 = _run(torch, msa, ctx, w, k, seed, cap_extra=cap_extra, fused=False)
    diff = float(np.max(np.abs(got - got2)))
    print(f"[gather_attn] max|O - O_two_calls| = {diff:.3e}", flush=True)
    assert diff <= 1e-2 * max(1.0, float(np.max(np.abs(ref))))


@pytest.mark.parametrize("cap_cut", [0, 30])
def test_gather_attn_one_token_invalid_ids_and_capacity(env, cap_cut):
    """Ids outside [0, n_docs) copy nothing and a capacity below the selected
    rows keeps the first cap_rows of them, as in msa_gather_device; the
    one-token call (the copy workgroups attending over their rows) then gives
    the rows, offsets and output of the two calls on the same arguments."""
    torch, msa, ctx = env
    seed, Hq, Hkv, L, rows, k = 940, 32, 8, 600, [90], 8
    w = P.peaked_inputs(seed, 1, 1, Hq, Hkv, D, L, rows, k, P.THETA)
    bank, coff, ids = _bank(w, k, seed)
    n_docs = len(coff) - 1
    ids = ids.copy()
    ids[0, 1] = n_docs + 5
    ids[0, 4] = -1
    valid = sorted(int(i) for i in ids[0] if 0 <= i < n_docs)
    want = int(sum(coff[i + 1] - coff[i] for i in valid))
    cap = want - cap_cut
    host = torch.empty(bank.shape, dtype=torch.bfloat16, pin_memory=True)
    host.copy_(W.dev_bf16(bank, "cpu"))
    coff_d, ids_d = torch.from_numpy(coff).cuda(), torch.from_numpy(ids).cuda()
    Q, Kl, Vl = W.dev_bf16(w["Q"]), W.dev_bf16(w["Kl"]), W.dev_bf16(w["Vl"])
    outs = []
    for fused in (True, False):
        dst = torch.full((cap, 2, Hkv, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        mo = torch.full((2,), -7, dtype=torch.int64, device="cuda")
        O = torch.full((1, 1, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        if fused:
            ws = msa.workspace(msa.msa_gather_attn_workspace_size(1, 1, 1, Hq, Hkv, k, cap, cap, L))
            msa.msa_gather_attn(ctx, host, 2 * Hkv * D * 2, bank.shape[0], coff_d, ids_d, dst, cap, mo, Q, cap, Kl,
                                Vl, k, w["scale"], O, ws)
        else:
            wsg = msa.workspace(msa.msa_gather_device_workspace_size(1, k, cap))
            msa.msa_gather_device(ctx, host, 2 * Hkv * D * 2, bank.shape[0], coff_d, ids_d, dst, cap, mo, wsg)
            wsa = msa.workspace(msa.msa_sparse_attn_workspace_size(1, 1, 1, Hq, Hkv, cap, L))
            msa.msa_sparse_attn(ctx, Q, dst, mo, cap, Kl, Vl, k, w["scale"], O, wsa)
        torch.cuda.synchronize()
        outs.append((W.host_bits(dst), mo.cpu().numpy(), W.widen(W.host_bits(O), "bf16")))
    (rows1, mo1, o1), (rows2, mo2, o2) = outs
    assert mo1.tolist() == mo2.tolist() == [0, cap]
    assert np.array_equal(rows1, rows2)
    ref_rows = np.concatenate([bank[coff[i]:coff[i + 1]] for i in valid])[:cap]
    assert np.array_equal(rows1, ref_rows)
    assert np.all(np.isfinite(o1))
    assert float(np.max(np.abs(o1 - o2))) <= 1e-2 * max(1.0, float(np.max(np.abs(o2))))


def test_gather_attn_fp32_takes_the_two_step_path(env):
    """fp32 (not on the fused path): the gather then the vector-unit attention, bar 1e-3."""
    torch, msa, ctx = env
    seed, B, Tq, Hq, Hkv, L, rows, k = 67, 2, 1, 32, 8, 300, [40, 90], 6
    w = P.peaked_inputs(seed, B, Tq, Hq, Hkv, D, L, rows, k, P.THETA)
    bank, coff, ids, got_rows, mo, got = _run(torch, msa, ctx, w, k, seed, dtype="f32")
    assert np.array_equal(mo, np.asarray(w["mem_off"], dtype=np.int64))
    P.assert_attn_close(got, P.oracle_out(w), 1e-3, "gather_attn fp32")


def test_gather_attn_one_query_past_the_single_launch_size(env):
    """One query with more than 8,192 memory rows: the plan + bounded copy
    beside the local keys, instead of the one-query copy."""
    torch, msa, ctx = env
    seed, B, Tq, Hq, Hkv, L, rows, k = 68, 1, 1, 32, 8, 64, [8300], 4
    w = P.peaked_inputs(seed, B, Tq, Hq, Hkv, D, L, rows, k, P.THETA)
    bank, coff, ids, got_rows, mo, got = _run(torch, msa, ctx, w, k, seed)
    assert mo.tolist() == [0, 8300]
    ref_rows, _ = oracle.gather_rows(bank, coff, ids[0])
    assert np.array_equal(oracle.f64_to_bf16_bits(got_rows[:8300]), ref_rows)
    P.assert_attn_close(got, P.oracle_out(w), 2e-2, "gather_attn 8,300 rows")


def test_gather_attn_spare_capacity(env):
    """A destination larger than the selected rows: mem_off ends at the rows
    actually gathered and the attention reads only those."""
    torch, msa, ctx = env
    seed, B, Tq, Hq, Hkv, L, rows, k = 69, 3, 1, 32, 8, 512, [20, 70, 33], 4
    w = P.peaked_inputs(seed, B, Tq, Hq, Hkv, D, L, rows, k, P.THETA)
    _, _, _, _, mo, got = _run(torch, msa, ctx, w, k, seed, cap_extra=500)
    assert np.array_equal(mo, np.asarray(w["mem_off"], dtype=np.int64))
    P.assert_attn_close(got, P.oracle_out(w), 2e-2, "gather_attn spare capacity")


def test_gather_attn_rejects_bad_arguments(env):
    torch, msa, ctx = env
    Hkv, Hq, L, k, cap = 8, 32, 64, 2, 16
    coff = torch.tensor([0, 4, 8, 12], dtype=torch.int64, device="cuda")
    host = torch.zeros((12, 2, Hkv, D), dtype=torch.bfloat16, pin_memory=True)
    ids = torch.tensor([[0, 2]], dtype=torch.int32, device="cuda")
    dst = torch.zeros((cap, 2, Hkv, D), dtype=torch.bfloat16, device="cuda")
    mo = torch.zeros(2, dtype=torch.int64, device="cuda")
    Q = torch.zeros((1, 1, Hq, D), dtype=torch.bfloat16, device="cuda")
    Kl = torch.zeros((1, L, Hkv, D), dtype=torch.bfloat16, device="cuda")
    O = torch.zeros_like(Q)
    need = msa.msa_gather_attn_workspace_size(1, 1, 1, Hq, Hkv, k, cap, 8, L)
    ws = msa.workspace(need)
    row_bytes = 2 * Hkv * D * 2
    with pytest.raises(msa.MsaError, match="row_bytes"):          # not one K̄ and one V̄ row
        msa.msa_gather_attn(ctx, host, row_bytes // 2, 12, coff, ids, dst, cap, mo, Q, 8, Kl, Kl, k, 0.1, O, ws)
    with pytest.raises(msa.MsaError) as e:                          # workspace too small
        msa.msa_gather_attn(ctx, host, row_bytes, 12, coff, ids, dst, cap, mo, Q, 8, Kl, Kl, k, 0.1, O,
                            ws[: max(need // 2, 256)])
    assert e.value.status == msa.MSA_ERR_WORKSPACE
    pageable = torch.zeros((12, 2, Hkv, D), dtype=torch.bfloat16)
    with pytest.raises(msa.MsaError, match="pinned"):
        msa.msa_gather_attn(ctx, pageable, row_bytes, 12, coff, ids, dst, cap, mo, Q, 8, Kl, Kl, k, 0.1, O, ws)
    with pytest.raises(msa.MsaError, match="max_pos"):
        msa.msa_gather_attn(ctx, host, row_bytes, 12, coff, ids, dst, cap, mo, Q, 8, Kl, Kl, 16380, 0.1, O, ws)
    torch.cuda.synchronize()
