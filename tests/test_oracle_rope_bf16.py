"""Pins of the oracle's bf16 conversion and RoPE against closed forms and
independent formulations (no GPU)."""

import math

import numpy as np
import pytest
import torch

import oracle


# ------------------------------------------------------------------ bf16

def test_bf16_roundtrip_all_finite_patterns():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    finite = bits[exp != 0xFF]
    x = oracle.bf16_bits_to_f64(finite)
    back = oracle.f64_to_bf16_bits(x)
    # +0 and -0 both map back to themselves
    assert np.array_equal(back, finite)


def test_bf16_round_half_to_even():
    one = 1.0
    ulp = 2.0 ** -7                      # bf16 spacing on [1, 2)
    # exactly halfway between 1 and 1+ulp -> even (1.0)
    assert oracle.f64_to_bf16_bits(np.array([one + ulp / 2]))[0] == 0x3F80
    # halfway between 1+ulp and 1+2ulp -> even (1+2ulp)
    assert oracle.f64_to_bf16_bits(np.array([one + 1.5 * ulp]))[0] == 0x3F82
    # just above halfway rounds up
    assert oracle.f64_to_bf16_bits(np.array([one + ulp / 2 + 1e-12]))[0] == 0x3F81
    assert oracle.f64_to_bf16_bits(np.array([-(one + 1.5 * ulp)]))[0] == 0xBF82


def test_bf16_matches_torch_cast_on_float32_values():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200000) * 10.0 ** rng.integers(-6, 6, 200000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f64_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------ RoPE

def test_inv_freq_closed_form():
    np.testing.assert_allclose(oracle.inv_freq(4, 1e4), [1.0, 1e-2], rtol=1e-15)
    np.testing.assert_allclose(oracle.inv_freq(8, 1e4), [1.0, 1e-1, 1e-2, 1e-3], rtol=1e-14)
    np.testing.assert_allclose(oracle.inv_freq(128, 1e6)[64 // 2], 1e6 ** -0.5, rtol=1e-14)


def test_rope_position_zero_is_identity_bitexact():
    x = np.random.default_rng(0).standard_normal((7, 3, 64))
    assert np.array_equal(oracle.rope(x, np.zeros((7, 1)), 1e4), x)


def test_rope_d2_is_plane_rotation_by_pos_radians():
    # d = 2: inv_freq_0 = 1, so position p rotates by p radians, counter-clockwise
    for p in [1, 2, 7, 100]:
        np.testing.assert_allclose(oracle.rope(np.array([1.0, 0.0]), p, 1e4),
                                   [math.cos(p), math.sin(p)], atol=1e-15)
        np.testing.assert_allclose(oracle.rope(np.array([0.0, 1.0]), p, 1e4),
                                   [-math.sin(p), math.cos(p)], atol=1e-15)


@pytest.mark.parametrize("theta", [1e4, 1e6])
def test_rope_equals_complex_multiplication(theta):
    rng = np.random.default_rng(1)
    d = 128
    x = rng.standard_normal((50, d))
    pos = rng.integers(0, 20000, size=50)
    got = oracle.rope(x, pos, theta)
    half = d // 2
    for r in range(50):
        for i in range(0, half, 7):
            z = complex(x[r, i], x[r, i + half]) * complex(
                math.cos(pos[r] * theta ** (-2 * i / d)), math.sin(pos[r] * theta ** (-2 * i / d)))
            assert abs(got[r, i] - z.real) < 1e-11
            assert abs(got[r, i + half] - z.imag) < 1e-11


def test_rope_preserves_norm_and_relative_positions():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for m, n, delta in [(3, 11, 5), (100, 2, 4000), (0, 8191, 17)]:
        a = oracle.rope(q, m, 1e6) @ oracle.rope(k, n, 1e6)
        b = oracle.rope(q, m + delta, 1e6) @ oracle.rope(k, n + delta, 1e6)
        assert abs(a - b) < 1e-10
        assert abs(np.linalg.norm(oracle.rope(q, m, 1e6)) - np.linalg.norm(q)) < 1e-12


def test_f32_widening_is_exact():
    # values with all 24 significand bits in use, and extremes of the range
    x = np.array([1 + 2.0 ** -23, -(2.0 ** 127) * (2 - 2.0 ** -23), 2.0 ** -149, 0.1], dtype=np.float32)
    w = oracle.f32_to_f64(x)
    assert w.dtype == np.float64
    assert w[0] == 1 + 2.0 ** -23 and w[1] == -(2.0 ** 127) * (2 - 2.0 ** -23) and w[2] == 2.0 ** -149
    assert w[3] == 0.100000001490116119384765625          # float32(0.1), not 0.1


def test_rope_angles_closed_form():
    # d = 4, theta = 100: inverse frequencies 1 and 1/10
    ang = oracle.rope_angles(np.array([0, 3, 7]), 4, 100.0)
    np.testing.assert_allclose(ang, [[0.0, 0.0], [3.0, 0.3], [7.0, 0.7]], rtol=1e-15, atol=0)
