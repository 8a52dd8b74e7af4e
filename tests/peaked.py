"""Attention inputs with a peaked softmax, for parity checks that can fail.

With N(0,1) queries and keys the softmax over a few thousand keys is nearly
flat and |O| is a few hundredths, so a kernel that shifts the global RoPE
offset k by one, drops half of the memory rows or skips the last local key
still lands within 2e-2 of the oracle.  These inputs plant a few keys per
checked query token so that they carry most of the softmax mass and |O| is of
order one:

* memory rows (used as stored, no rotation inside the attention) aligned with
  the high-frequency rotary pairs of the token's query rotated to its global
  position k + (L - Tq) + i: the first and last row of the query's memory
  range and two rows in each half; the product depends on that position, so
  an offset error of one position moves their logits by several units;
* the local key on the token's own position (same rotation on both sides,
  so it is aligned with the unrotated query);
* the local key seven positions back, aligned with the high-frequency pairs
  of the query rotated by seven positions (the relative offset), so a local
  position error of one moves its logit as well.

Everything else stays N(0,1), and the values are scaled by 1/4, so that the
largest output element is about one.  On such inputs a bf16 kernel's own
rounding of the rotated query and local keys (2^-9 relative per element)
moves a planted logit of 10 by a few hundredths, which shifts the output by
under 1% of max|O| (a CPU emulation of that rounding gives 0.4-0.9% on these
shapes); the mistakes above move it by 35% or more.

The queries are drawn first and the planted
keys are built from them with the oracle's RoPE (test infrastructure; the
HIP path is never consulted), then rounded to bf16, so both sides read the
same bits.  The reading of the pages these inputs exercise is the neo-ai.one
MSA article's global RoPE (全体設計 › アーキテクチャ, Fig. 2): memory keys
carry document-local positions and the query starts at offset k.
"""

import numpy as np

import msa_synth
import oracle

N_HF = 8            # rotary pairs counted as high-frequency (inverse frequency >= theta^(-14/128))
LOCAL_BACK = 7      # distance of the second planted local key
V_SCALE = 0.25      # values are N(0,1) / 4, so the output's largest element is about one


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _hf_mask(d):
    m = np.zeros(d)
    m[:N_HF] = 1.0
    m[d // 2:d // 2 + N_HF] = 1.0
    return m


def _group_dir(vecs, G):
    """[Hq, d] -> [Hkv, d]: unit direction of the sum of each group's unit vectors."""
    Hq, d = vecs.shape
    return _unit(_unit(vecs).reshape(Hq // G, G, d).sum(axis=1))


def memory_plant_rows(rows_b):
    """The planted positions inside a query's memory range of rows_b rows:
    its first and last row and two more in each half (fewer for tiny ranges)."""
    if rows_b <= 0:
        return []
    return sorted({0, rows_b - 1} | {int(f * rows_b) for f in (0.125, 0.375, 0.625, 0.875)})


def _aimed(target_dir, qs, logit, scale):
    """Key of direction target_dir [d] scaled so that the mean over the group's
    query vectors qs [G, d] of scale * q.k equals `logit`."""
    proj = float(np.mean(qs @ target_dir))
    assert proj > 0.0, "a planted direction must point along its group's queries"
    return logit * target_dir / (scale * proj)


def aim_memory_keys(q_tok, pos, theta, G, logit=10.0):
    """Memory keys [Hkv, d] (used as stored) whose product with the query
    q_tok [Hq, d] rotated to global position `pos` has a mean logit of `logit`
    over each group's heads, built on the high-frequency rotary pairs."""
    Hq, d = q_tok.shape
    scale = 1.0 / np.sqrt(d)
    qrot = oracle.rope(q_tok, np.full(Hq, pos), theta)
    dirs = _group_dir(qrot * _hf_mask(d), G)
    return np.stack([_aimed(dirs[g], qrot[g * G:(g + 1) * G], logit, scale) for g in range(Hq // G)])


def aim_local_keys(q_tok, back, theta, G, logit=10.0):
    """Unrotated local keys [Hkv, d] placed `back` positions before the query
    token q_tok [Hq, d] with a mean logit of `logit` over each group's heads
    (back = 0: the token's own key, aligned with the unrotated query; else
    along the high-frequency pairs of the query rotated by `back`)."""
    Hq, d = q_tok.shape
    scale = 1.0 / np.sqrt(d)
    if back == 0:
        dirs, qs = _group_dir(q_tok, G), q_tok
    else:
        qs = oracle.rope(q_tok, np.full(Hq, back), theta)
        dirs = _group_dir(qs * _hf_mask(d), G)
    return np.stack([_aimed(dirs[g], qs[g * G:(g + 1) * G], logit, scale) for g in range(Hq // G)])


def peaked_inputs(seed, B, Tq, Hq, Hkv, d, L, rows, qoff, theta, tokens=None, logit=10.0):
    """bf16 bits of Q [B,Tq,Hq,d], KV [M,2,Hkv,d], K_loc, V_loc [B,L,Hkv,d]
    and int64 mem_off [B+1], with keys planted for the query tokens in
    `tokens` (default: the last token) of every query, each planted key at a
    mean logit of `logit` over its group's query heads.  Returns a dict."""
    G = Hq // Hkv
    mem_off = msa_synth.prefix_offsets(rows)
    M = int(mem_off[-1])
    tokens = [Tq - 1] if tokens is None else list(tokens)
    Q = msa_synth.normal_bf16(seed, 1, (B, Tq, Hq, d))
    KV = msa_synth.normal_bf16(seed, 2, (max(M, 1), 2, Hkv, d))
    Kl = msa_synth.normal_bf16(seed, 3, (B, L, Hkv, d))
    Vl = msa_synth.normal_bf16(seed, 4, (B, L, Hkv, d))
    q64 = oracle.bf16_bits_to_f64(Q)
    kv64 = oracle.bf16_bits_to_f64(KV[:, 0])
    kl64 = oracle.bf16_bits_to_f64(Kl)
    for b in range(B):
        nb = int(mem_off[b + 1] - mem_off[b])
        slots = memory_plant_rows(nb)
        for n, i in enumerate(tokens):
            j = (L - Tq) + i
            mem = aim_memory_keys(q64[b, i], qoff + j, theta, G, logit)
            for s in slots[n::len(tokens)]:
                kv64[mem_off[b] + s] = mem
            kl64[b, j] = aim_local_keys(q64[b, i], 0, theta, G, logit)
            if j - LOCAL_BACK >= 0:
                kl64[b, j - LOCAL_BACK] = aim_local_keys(q64[b, i], LOCAL_BACK, theta, G, logit)
    KV[:, 0] = oracle.f64_to_bf16_bits(kv64)
    Kl = oracle.f64_to_bf16_bits(kl64)
    # values scaled by 1/4 (exact in bf16) so that |O| stays near one
    KV[:, 1] = oracle.f64_to_bf16_bits(V_SCALE * oracle.bf16_bits_to_f64(KV[:, 1]))
    Vl = oracle.f64_to_bf16_bits(V_SCALE * oracle.bf16_bits_to_f64(Vl))
    return dict(Q=Q, KV=KV, Kl=Kl, Vl=Vl, mem_off=mem_off, tokens=tokens, qoff=qoff, theta=theta,
                scale=1.0 / np.sqrt(d))


def oracle_out(w, qoff=None, mem_keep=None, drop_last_local=False, local_shift=0, mem_late=False):
    """The oracle on peaked inputs, optionally with one deliberate mistake
    (the negative controls): another RoPE offset, only the first mem_keep
    fraction of every query's memory rows, the query token's own local key
    made invisible, every local key rotated local_shift positions further, or
    every query's memory range read one row late (its first row missed, the
    row after its range, a zero row past the buffer's end, read instead)."""
    Q = oracle.bf16_bits_to_f64(w["Q"])
    kv = oracle.bf16_bits_to_f64(w["KV"])
    Kl = oracle.bf16_bits_to_f64(w["Kl"])
    Vl = oracle.bf16_bits_to_f64(w["Vl"])
    mem_off = np.asarray(w["mem_off"], dtype=np.int64)
    B, Tq, Hq, d = Q.shape
    L = Kl.shape[1]
    mK, mV = kv[:, 0], kv[:, 1]
    if mem_keep is not None:
        parts_k, parts_v, off = [], [], [0]
        for b in range(B):
            a, e = int(mem_off[b]), int(mem_off[b + 1])
            e2 = a + int((e - a) * mem_keep)
            parts_k.append(mK[a:e2])
            parts_v.append(mV[a:e2])
            off.append(off[-1] + e2 - a)
        mK, mV, mem_off = np.concatenate(parts_k), np.concatenate(parts_v), np.array(off)
    if mem_late:
        M = int(mem_off[-1])
        padK = np.concatenate([mK[:M], np.zeros((1,) + mK.shape[1:])])
        padV = np.concatenate([mV[:M], np.zeros((1,) + mV.shape[1:])])
        idx = np.concatenate([np.arange(mem_off[b] + 1, mem_off[b + 1] + 1) for b in range(B)]
                             + [np.zeros(0, dtype=np.int64)])
        mK, mV = padK[idx], padV[idx]
    if drop_last_local:
        # a key whose logit is about -1e4 for every query head of its group has weight 0
        G = Hq // Kl.shape[2]
        Kl = Kl.copy()
        for b in range(B):
            for i in w["tokens"]:
                Kl[b, (L - Tq) + i] = -1e4 * _group_dir(Q[b, i], G)
    if local_shift:
        Kl = oracle.rope(Kl, np.full(Kl.shape[:-1], local_shift), w["theta"])
    return oracle.sparse_attn(Q, mK, mV, mem_off, Kl, Vl, w["qoff"] if qoff is None else qoff,
                              w["scale"], w["theta"])


def token_view(w, i):
    """The inputs one query token i of a prefill (Tq == L) sees: its own query
    row and local keys 0..i, as a one-token query of L = i + 1 (the token
    keeps its global position k + i)."""
    assert w["Q"].shape[1] == w["Kl"].shape[1], "token_view needs Tq == L"
    v = dict(w)
    v.update(Q=w["Q"][:, i:i + 1], Kl=w["Kl"][:, :i + 1], Vl=w["Vl"][:, :i + 1], tokens=[0])
    return v


def assert_attn_close(got, ref, tol, what=""):
    """The attention bar: max|O - O_ref| <= tol, and also <= tol * max|O_ref|
    (the error measured against the output's own size, so a nearly flat
    softmax with a small |O| cannot hide an error).  Prints both numbers."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    peak = float(np.max(np.abs(ref))) if ref.size else 0.0
    rel = err / peak if peak > 0 else (0.0 if err == 0 else float("inf"))
    print(f"[attn] {what} max-abs {err:.3e}  max|O_ref| {peak:.3e}  ratio {rel:.3e}", flush=True)
    assert err <= tol, f"{what}: max-abs {err:.3e} > {tol}"
    assert err <= tol * peak, f"{what}: max-abs {err:.3e} > {tol} * max|O_ref| = {tol * peak:.3e}"
    return err, rel


# Shapes of the peaked parity cases (GPU) and of their negative controls (CPU):
# seed, B, Tq, Hq, Hkv, L, memory rows per query, k.  Head dim 128, theta 1e6.
DECODE_CASES = [
    (31, 1, 1, 32, 8, 2048, [125], 16),                # the 100M-token step's decode shape
    (32, 1, 1, 32, 8, 8192, [1000], 16),               # long local context, many memory rows
    (33, 4, 1, 32, 8, 2048, [125, 0, 400, 37], 16),    # a batch, one query without memory
    (34, 2, 1, 8, 8, 3000, [200, 90], 16),             # G = 1
    (35, 2, 1, 64, 8, 1500, [300, 60], 16),            # G = 8
    (36, 1, 4, 32, 8, 2048, [250], 32),                # four query tokens, each planted
]
# 8K prefill over 250 memory rows: tokens 4095 and 8191 planted and checked
PREFILL_CASE = dict(seed=37, T=8192, M=250, qoff=32, tokens=(4095, 8191))
THETA = 1e6
