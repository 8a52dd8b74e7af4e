"""bfloat16 <-> float64 for the oracle (test infrastructure only).

bf16 tensors are held as their raw uint16 bit patterns.  Widening is exact
(bf16 is the top half of an IEEE binary32).  Narrowing rounds once, to
nearest-even, from float64 directly (no float32 intermediate), so the oracle
rounds exactly once wherever it emits a stored bf16 value.

Pinned by tests/test_oracle_bf16.py: exact round trip of every finite bf16
pattern, halfway cases rounding to even, and agreement with torch's own
float32->bfloat16 cast on values that are exactly representable in float32.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """uint16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f32_to_f64(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """float64 -> uint16 bf16 bits, round to nearest, ties to even.

    Works on the exact binary value of x: the bf16 grid spacing at x is
    2**(e-7) for x in [2**e, 2**(e+1)); x is divided into an integer multiple
    of that spacing with np.rint (which rounds half to even), then rebuilt.
    Finite inputs only; overflow saturates to +-inf as IEEE rounding does.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    ax = np.abs(x)
    nz = ax > 0
    # exponent of the leading bit; bf16 normal range uses 8 significant bits,
    # subnormals have a fixed spacing of 2**-133.
    e = np.zeros(x.shape, dtype=np.int64)
    e[nz] = np.floor(np.log2(ax[nz])).astype(np.int64)
    # guard against log2 rounding at exact powers of two
    too_big = nz & (np.ldexp(1.0, e) > ax)
    e[too_big] -= 1
    too_small = nz & (np.ldexp(1.0, e + 1) <= ax)
    e[too_small] += 1
    e = np.maximum(e, -126)
    spacing_exp = e - 7
    q = np.rint(np.ldexp(x, -spacing_exp))
    out[:] = np.ldexp(q, spacing_exp)
    out[~nz] = x[~nz]
    out = np.where(np.abs(out) >= 2.0 ** 128, np.copysign(np.inf, out), out)
    f32 = out.astype(np.float32)  # exact: every bf16 value is a binary32 value
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
