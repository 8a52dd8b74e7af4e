"""Writes tests/golden/tiny_route_attn.json from the oracle alone.

The pages about MSA print no worked numerical example (no pooled tensor,
score or attention output), so nothing here is the pages' own number.  This
fixture freezes the oracle's answer on one tiny seeded case so that a later
change to the oracle's arithmetic shows up as a failing regression test and
must be justified by the passage it follows.  Inputs come from msa_synth;
expected values come only from oracle/.

Run:  python tests/golden/make_golden.py
"""

import json
import math
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import msa_synth  # noqa: E402
import oracle     # noqa: E402

CASE = dict(seed=11, lengths=[5, 9, 3, 16, 7], chunk_len=4, Hq=4, Hkv=2, d=8,
            Tq=2, L=3, top_k=2, theta=10000.0)


def inputs(c):
    T = sum(c["lengths"])
    H, d = c["Hkv"], c["d"]
    K = msa_synth.normal_f32(c["seed"], 1, (T, H, d)).astype(np.float64)
    V = msa_synth.normal_f32(c["seed"], 2, (T, H, d)).astype(np.float64)
    Kr = msa_synth.normal_f32(c["seed"], 3, (T, H, d)).astype(np.float64)
    Qr = msa_synth.normal_f32(c["seed"], 4, (1, c["Tq"], c["Hq"], d)).astype(np.float64)
    Q = msa_synth.normal_f32(c["seed"], 5, (1, c["Tq"], c["Hq"], d)).astype(np.float64)
    Kl = msa_synth.normal_f32(c["seed"], 6, (1, c["L"], H, d)).astype(np.float64)
    Vl = msa_synth.normal_f32(c["seed"], 7, (1, c["L"], H, d)).astype(np.float64)
    return K, V, Kr, Qr, Q, Kl, Vl


def expected(c):
    K, V, Kr, Qr, Q, Kl, Vl = inputs(c)
    off = msa_synth.prefix_offsets(c["lengths"])
    Kb, Vb, Rb = oracle.encode_pool(K, V, Kr, off, c["chunk_len"], c["theta"])
    coff = oracle.chunk_offsets(off, c["chunk_len"])
    ids, sc, cs, D = oracle.route(Qr, Rb, coff, c["top_k"])
    mK, m = oracle.gather_rows(Kb, coff, ids[0])
    mV, _ = oracle.gather_rows(Vb, coff, ids[0])
    O = oracle.sparse_attn(Q, mK, mV, [0, m], Kl, Vl, c["top_k"], 1 / math.sqrt(c["d"]), c["theta"])
    return dict(Kbar=Kb, Vbar=Vb, Krbar=Rb, chunk_scores=cs, doc_scores=D,
                ids=ids, top_scores=sc, O=O)


if __name__ == "__main__":
    out = {k: np.asarray(v).tolist() for k, v in expected(CASE).items()}
    out["case"] = CASE
    with open(os.path.join(HERE, "tiny_route_attn.json"), "w") as f:
        json.dump(out, f, indent=None, separators=(",", ":"))
    print("wrote tiny_route_attn.json")
