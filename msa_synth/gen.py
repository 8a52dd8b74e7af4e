"""Seeded input generators (no method arithmetic; see package docstring)."""

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_STREAM_MUL = np.uint64(0xD1B54A32D192ED03)


# ---------------------------------------------------------------- dtype bits

def f32_to_bf16_bits(x):
    """float32 -> bf16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits):
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- PCG64 normals

def _rng(seed, stream):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream)])))


def normal_f32(seed, stream, shape):
    """Standard normals (PCG64 keyed by (seed, stream)), rounded to float32."""
    return _rng(seed, stream).standard_normal(shape).astype(np.float32)


def normal_bf16(seed, stream, shape):
    """Standard normals drawn in float32 (PCG64 keyed by (seed, stream)),
    rounded to bf16 bits (uint16)."""
    return f32_to_bf16_bits(_rng(seed, stream).standard_normal(shape, dtype=np.float32))


# ---------------------------------------------------------------- counter-based

def _mix(z):
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64_key(seed, stream):
    """State of the stream: mix(mix(seed) xor (stream * 0xD1B54A32D192ED03))."""
    with np.errstate(over="ignore"):
        s = _mix(np.array([seed], dtype=np.uint64))
        k = _mix(s ^ (np.array([stream], dtype=np.uint64) * _STREAM_MUL))
    return int(k[0])


def _counter_codes(seed, stream, start, count):
    key = np.uint64(splitmix64_key(seed, stream))
    idx = np.arange(start, start + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = _mix(key + (idx + np.uint64(1)) * _GOLDEN)
    m = np.uint64(63)
    s = (z & m) + ((z >> np.uint64(6)) & m) + ((z >> np.uint64(12)) & m) + ((z >> np.uint64(18)) & m)
    return s.astype(np.int32) - 126          # in [-126, 126]


def counter_f32(seed, stream, start, count):
    """Elements start .. start+count-1 of the stream as float32 values k/32."""
    return (_counter_codes(seed, stream, start, count).astype(np.float32) / np.float32(32.0))


def counter_bf16(seed, stream, start, count):
    """Same values as bf16 bits (exact: |k| <= 126 needs at most 7 bits)."""
    f = counter_f32(seed, stream, start, count)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------- documents

def uniform_lengths(seed, n_docs, lo, hi):
    """Integer document lengths uniform on [lo, hi]."""
    return _rng(seed, 0x1E9).integers(lo, hi + 1, size=n_docs).astype(np.int64)


def lognormal_lengths(seed, total_tokens, median=400.0, sigma=0.67,
                      lo=64, hi=8192, multiple=64):
    """Log-normal lengths (given median and log-sd), clipped to [lo, hi] and
    rounded to a multiple of `multiple`, drawn until total_tokens is reached;
    the last document is truncated so the lengths sum to total_tokens.
    total_tokens must be a multiple of `multiple`."""
    if total_tokens % multiple:
        raise ValueError("total must be a multiple of the rounding unit")
    rng = _rng(seed, 0x10C)
    out = []
    acc = 0
    while acc < total_tokens:
        draw = rng.lognormal(np.log(median), sigma, size=65536)
        draw = np.clip(draw, lo, hi)
        draw = (np.rint(draw / multiple) * multiple).astype(np.int64)
        draw = np.clip(draw, lo, hi)
        cs = acc + np.cumsum(draw)
        n_take = int(np.searchsorted(cs, total_tokens, side="left")) + 1
        n_take = min(n_take, len(draw))
        take = draw[:n_take].copy()
        new_acc = acc + int(take.sum())
        if new_acc >= total_tokens:
            take[-1] -= new_acc - total_tokens
            if take[-1] == 0:
                take = take[:-1]
            out.append(take)
            acc = total_tokens
        else:
            out.append(take)
            acc = new_acc
    return np.concatenate(out).astype(np.int64)


def prefix_offsets(lengths):
    """[0, l0, l0+l1, ...] as int64."""
    lengths = np.asarray(lengths, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


def ceil_chunk_offsets(lengths, chunk_len):
    """Row layout of a bank that is synthesised already pooled: document d
    owns rows [off[d], off[d+1]) with off the prefix sum of ceil(len/c)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    return prefix_offsets((lengths + chunk_len - 1) // chunk_len)


# ---------------------------------------------------------------- planting

def pick_planted(seed, stream, n_docs, n_planted, exclude=()):
    """Distinct document ids, seeded, none in `exclude`."""
    rng = _rng(seed, stream)
    excl = set(int(e) for e in exclude)
    cand = np.array([i for i in rng.permutation(n_docs)[: n_planted + len(excl)]
                     if int(i) not in excl][:n_planted], dtype=np.int64)
    if len(cand) < n_planted:
        raise ValueError("not enough documents to plant")
    return np.sort(cand)


def planted_rows(seed, stream, q_token, n_kv_heads, n_rows, weight=0.8, noise=0.6,
                 out="bf16"):
    """Rows made to point at one query token: for KV head g,

        row[g] = weight * u_g + noise * eps,   u_g = sum_{h in group g} q_h / sqrt(G)

    with q_token [Hq, d] float (the query token's stored values), G = Hq / Hkv
    and eps standard normal (PCG64 keyed by (seed, stream)), fresh per row.
    For G = 1 this is the literal `weight * q + noise * noise` recipe.
    Returned as bf16 bits (out='bf16') or float32 (out='f32'), rounded once."""
    q = np.asarray(q_token, dtype=np.float64)
    Hq, d = q.shape
    G = Hq // n_kv_heads
    u = q.reshape(n_kv_heads, G, d).sum(axis=1) / np.sqrt(G)      # [Hkv, d]
    eps = _rng(seed, stream).standard_normal((n_rows, n_kv_heads, d))
    rows = weight * u[None] + noise * eps
    f = rows.astype(np.float32)
    return f32_to_bf16_bits(f) if out == "bf16" else f
