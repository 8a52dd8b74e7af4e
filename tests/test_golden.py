"""The oracle still reproduces its frozen tiny case (regression pin)."""

import json
import os

import numpy as np

from tests.golden.make_golden import CASE, expected

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_oracle_reproduces_frozen_case():
    with open(os.path.join(HERE, "tiny_route_attn.json")) as f:
        gold = json.load(f)
    assert gold["case"] == CASE
    got = expected(CASE)
    for key, val in got.items():
        np.testing.assert_allclose(np.asarray(val, dtype=np.float64), np.asarray(gold[key]),
                                   rtol=1e-12, atol=1e-13, err_msg=key)
