"""Negative controls for the attention parity bar (CPU, oracle only).

On the peaked inputs of tests/peaked.py the GPU parity tests require
max|O - O_ref| <= 2e-2 and <= 2e-2 * max|O_ref| in bf16.  Here the oracle
itself is run with one plausible kernel mistake at a time, on the same
shapes and seeds; each mistaken output must violate that bar, so a kernel
that made the mistake could not pass.  Mistakes: the global RoPE offset k
off by one either way (neo-ai.one MSA article, 全体設計 › アーキテクチャ:
the query start moves by k), half of the memory rows dropped, the token's
own local key skipped, every local key one position off, and the memory
range read one row late.
"""

import numpy as np
import pytest

from tests import peaked as P

TOL = 2e-2


def _violates(bad, ref):
    err = float(np.max(np.abs(bad - ref)))
    peak = float(np.max(np.abs(ref)))
    return err > TOL * peak and err > TOL, (err, peak)


def _mistakes(w):
    yield "k+1", P.oracle_out(w, qoff=w["qoff"] + 1)
    yield "k-1", P.oracle_out(w, qoff=w["qoff"] - 1)
    yield "half the memory rows", P.oracle_out(w, mem_keep=0.5)
    yield "own local key skipped", P.oracle_out(w, drop_last_local=True)
    yield "local keys one position off", P.oracle_out(w, local_shift=1)
    if int(w["mem_off"][-1]) > 0:
        yield "memory range one row late", P.oracle_out(w, mem_late=True)


@pytest.mark.parametrize("seed,B,Tq,Hq,Hkv,L,rows,qoff", P.DECODE_CASES)
def test_decode_mistakes_fail_the_bar(seed, B, Tq, Hq, Hkv, L, rows, qoff):
    w = P.peaked_inputs(seed, B, Tq, Hq, Hkv, 128, L, rows, qoff, P.THETA,
                        tokens=list(range(Tq)))
    ref = P.oracle_out(w)
    assert np.max(np.abs(ref)) > 0.25          # peaked: |O| of order one
    for name, bad in _mistakes(w):
        ok, (err, peak) = _violates(bad, ref)
        assert ok, f"{name}: max-abs {err:.3e} vs max|O_ref| {peak:.3e} passes the bar"


def test_prefill_mistakes_fail_the_bar_at_the_checked_tokens():
    c = P.PREFILL_CASE
    w = P.peaked_inputs(c["seed"], 1, c["T"], 32, 8, 128, c["T"], [c["M"]], c["qoff"], P.THETA,
                        tokens=c["tokens"])
    for i in c["tokens"]:
        v = P.token_view(w, i)
        ref = P.oracle_out(v)
        assert np.max(np.abs(ref)) > 0.25
        for name, bad in _mistakes(v):
            ok, (err, peak) = _violates(bad, ref)
            assert ok, f"token {i}, {name}: max-abs {err:.3e} vs max|O_ref| {peak:.3e} passes the bar"


def test_bar_accepts_bf16_rounding_of_the_oracle_output():
    # the bar itself is not stricter than storing the exact result in bf16
    import oracle
    w = P.peaked_inputs(*P.DECODE_CASES[0][:5], 128, *P.DECODE_CASES[0][5:], P.THETA)
    ref = P.oracle_out(w)
    stored = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(ref))
    P.assert_attn_close(stored, ref, TOL, "bf16-rounded oracle")
