"""Seeded workloads shared by the GPU parity tests, smoke() and bench.py.

Inputs come only from msa_synth; expected values come only from oracle/.
This module never computes any part of the method: it lays inputs out and
moves bits between host and device.
"""

import math

import numpy as np

import msa_synth

# Qwen3-4B-shaped routing layer: 32 query heads, 8 KV heads, head dim 128
QWEN_HQ, QWEN_HKV, QWEN_D = 32, 8, 128


# ---------------------------------------------------------------- bits <-> torch

def dev_bf16(bits, device="cuda"):
    import torch
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)


def dev_f32(x, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def host_bits(t):
    """bf16 torch tensor -> uint16 numpy bits; f32 -> float32 numpy."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def dev(x, dtype, device="cuda"):
    return dev_bf16(x, device) if dtype == "bf16" else dev_f32(x, device)


def draw(seed, stream, shape, dtype):
    """Standard normals in the storage dtype (bits for bf16)."""
    return msa_synth.normal_bf16(seed, stream, shape) if dtype == "bf16" else \
        msa_synth.normal_f32(seed, stream, shape)


def widen(x, dtype):
    """Storage values -> float64 for the oracle (widening is exact)."""
    import oracle
    return oracle.bf16_bits_to_f64(x) if dtype == "bf16" else oracle.f32_to_f64(x)


def round_store(x64, dtype):
    """float64 oracle result rounded once to the storage dtype, widened back."""
    import oracle
    if dtype == "bf16":
        return oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(x64))
    return np.asarray(x64, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------- pooled banks

def pooled_bank_krbar(seed, layer, N, Hkv, d):
    """Counter-generated pooled routing keys of one layer, bf16 bits [N, Hkv, d]."""
    return msa_synth.counter_bf16(seed, 1000 + layer, 0, N * Hkv * d).reshape(N, Hkv, d)


def krbar_stream(layer):
    return 1000 + layer


def kvbar_stream(layer):
    return 5000 + layer


def planted_pooled(seed, layer, qr_token, Hkv, n_rows, tag=0):
    """Pooled K̄r rows of a planted document (bf16 bits [n_rows, Hkv, d])."""
    return msa_synth.planted_rows(seed, 9000 + 97 * layer + tag, qr_token, Hkv, n_rows)


def tiny_fp32(seed=0):
    """64 documents x 256 tokens, chunk 16, Hq 4 / Hkv 2, d 64, fp32; raw
    K, V, Kr, Qr, Q, local K/V ~ N(0,1); 4 planted documents whose raw Kr rows
    are 0.8 u + 0.6 noise for a random query token; 32 local query tokens;
    top-k 4."""
    Hq, Hkv, d, c, T_q, L, k = 4, 2, 64, 16, 32, 32, 4
    lens = np.full(64, 256, dtype=np.int64)
    tok = msa_synth.prefix_offsets(lens)
    T = int(tok[-1])
    w = dict(dtype="f32", Hq=Hq, Hkv=Hkv, d=d, chunk=c, Tq=T_q, L=L, top_k=k, theta=1e4,
             lens=lens, tok_off=tok, n_docs=64)
    w["K"] = msa_synth.normal_f32(seed, 1, (T, Hkv, d))
    w["V"] = msa_synth.normal_f32(seed, 2, (T, Hkv, d))
    Kr = msa_synth.normal_f32(seed, 3, (T, Hkv, d))
    w["Qr"] = msa_synth.normal_f32(seed, 4, (1, T_q, Hq, d))
    w["Q"] = msa_synth.normal_f32(seed, 5, (1, T_q, Hq, d))
    w["K_loc"] = msa_synth.normal_f32(seed, 6, (1, L, Hkv, d))
    w["V_loc"] = msa_synth.normal_f32(seed, 7, (1, L, Hkv, d))
    planted = msa_synth.pick_planted(seed, 50, 64, 4)
    toks = np.random.default_rng(seed + 51).integers(0, T_q, size=4)
    for j, doc in enumerate(planted):
        Kr[tok[doc]:tok[doc + 1]] = msa_synth.planted_rows(seed, 60 + j, w["Qr"][0, toks[j]], Hkv,
                                                           int(lens[doc]), out="f32")
    w["Kr"] = Kr
    w["planted"] = planted
    return w


def qwen_bf16_layer(seed=0, n_docs=2000, lo=128, hi=1024, Tq=256, top_k=16, n_planted=16):
    """One Qwen3-4B-shaped routing layer in bf16: n_docs documents with integer
    lengths uniform in [lo, hi], chunk 64; raw Kr ~ N(0,1) (PCG64) with
    n_planted documents planted against random query tokens; raw K and V
    from the counter generator (filled on the device; the oracle regenerates
    the rows it needs); Qr of Tq tokens; a 1-token decode query (Q, local
    K/V of L = Tq + 1 tokens, the decode token last)."""
    Hq, Hkv, d, c = QWEN_HQ, QWEN_HKV, QWEN_D, 64
    lens = msa_synth.uniform_lengths(seed, n_docs, lo, hi)
    tok = msa_synth.prefix_offsets(lens)
    T = int(tok[-1])
    L = Tq + 1
    w = dict(dtype="bf16", Hq=Hq, Hkv=Hkv, d=d, chunk=c, Tq=Tq, L=L, top_k=top_k, theta=1e6,
             lens=lens, tok_off=tok, n_docs=n_docs, T=T, seed=seed)
    Qr = msa_synth.normal_bf16(seed, 4, (1, Tq, Hq, d))
    Kr = msa_synth.normal_bf16(seed, 3, (T, Hkv, d))
    planted = msa_synth.pick_planted(seed, 50, n_docs, n_planted)
    toks = np.random.default_rng(seed + 51).integers(0, Tq, size=n_planted)
    qf = msa_synth.bf16_bits_to_f32(Qr)
    for j, doc in enumerate(planted):
        Kr[tok[doc]:tok[doc + 1]] = msa_synth.planted_rows(seed, 60 + j, qf[0, toks[j]], Hkv,
                                                           int(lens[doc]))
    w.update(Qr=Qr, Kr=Kr, planted=planted)
    w["Q"] = msa_synth.normal_bf16(seed, 5, (1, 1, Hq, d))
    w["K_loc"] = msa_synth.normal_bf16(seed, 6, (1, L, Hkv, d))
    w["V_loc"] = msa_synth.normal_bf16(seed, 7, (1, L, Hkv, d))
    w["K_stream"], w["V_stream"] = 11, 12   # counter streams of raw K and V
    return w


def counter_bf16_threads(seed, stream, start, count, threads=16, block=1 << 23):
    """msa_synth.counter_bf16 over [start, start+count), evaluated on slices by
    a thread pool (NumPy releases the GIL inside its ufuncs)."""
    from concurrent.futures import ThreadPoolExecutor
    out = np.empty(count, dtype=np.uint16)

    def job(o):
        n = min(block, count - o)
        out[o:o + n] = msa_synth.counter_bf16(seed, stream, start + o, n)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(job, range(0, count, block)))
    return out


def counter_rows(seed, stream, row0, row1, Hkv, d):
    """Rows row0..row1-1 of a counter-filled [T, Hkv, d] bf16 tensor."""
    n = Hkv * d
    return msa_synth.counter_bf16(seed, stream, row0 * n, (row1 - row0) * n).reshape(-1, Hkv, d)


def rel_row_err(got, ref):
    """max over rows of |got - ref| / (|ref| + rms(ref row)), rows = last axis."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    return float(np.max(np.abs(got - ref) / (np.abs(ref) + rms + 1e-300)))


def scale_of(d):
    return 1.0 / math.sqrt(d)
