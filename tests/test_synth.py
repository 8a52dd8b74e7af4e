"""Checks of the seeded input generators (no GPU)."""

import numpy as np

import msa_synth


def test_normals_are_seeded_and_streams_differ():
    a = msa_synth.normal_bf16(0, 1, (100,))
    assert np.array_equal(a, msa_synth.normal_bf16(0, 1, (100,)))
    assert not np.array_equal(a, msa_synth.normal_bf16(0, 2, (100,)))
    assert not np.array_equal(a, msa_synth.normal_bf16(1, 1, (100,)))


def test_f32_to_bf16_is_round_to_nearest_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8) - 2 ** -20], np.float32)
    assert msa_synth.f32_to_bf16_bits(x).tolist() == [0x3F80, 0x3F82, 0xBF81]


def test_counter_values_are_exact_in_bf16_and_slices_agree():
    full = msa_synth.counter_f32(7, 3, 0, 10000)
    bits = msa_synth.counter_bf16(7, 3, 0, 10000)
    assert np.array_equal(msa_synth.bf16_bits_to_f32(bits), full)
    assert np.array_equal(msa_synth.counter_bf16(7, 3, 1234, 500), bits[1234:1734])
    k = full * 32
    assert np.array_equal(k, np.rint(k)) and np.abs(k).max() <= 126


def test_counter_distribution():
    x = msa_synth.counter_f32(1, 0, 0, 1 << 20).astype(np.float64)
    assert abs(x.mean()) < 0.01
    assert abs(x.std() - np.sqrt(4 * (64 ** 2 - 1) / 12) / 32) < 0.01


def test_splitmix64_first_outputs_of_published_definition():
    # SplitMix64 output i from state s is mix(s + i * 0x9E3779B97F4A7C15).
    # With state 0 the first output is the published constant 0xE220A8397B1DCDAF.
    key = 0
    M = (1 << 64) - 1
    z = (key + 0x9E3779B97F4A7C15) & M
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M
    z ^= z >> 31
    assert z == 0xE220A8397B1DCDAF


def test_lognormal_lengths_recipe():
    lens = msa_synth.lognormal_lengths(0, 10_000_000)
    assert lens.sum() == 10_000_000
    assert np.all(lens % 64 == 0) and lens.min() >= 64 and lens.max() <= 8192
    assert 17_000 < len(lens) < 23_000
    assert 350 <= np.median(lens) <= 450


def test_uniform_lengths_and_offsets():
    lens = msa_synth.uniform_lengths(0, 2000, 128, 1024)
    assert lens.min() >= 128 and lens.max() <= 1024
    off = msa_synth.prefix_offsets(lens)
    assert off[0] == 0 and off[-1] == lens.sum()
    coff = msa_synth.ceil_chunk_offsets(lens, 64)
    assert coff[-1] == int(np.sum((lens + 63) // 64))


def test_planted_rows_follow_recipe_for_one_group():
    q = np.random.default_rng(0).standard_normal((2, 16)).astype(np.float32)
    rows = msa_synth.planted_rows(5, 9, q, 2, 3, out="f32")     # G = 1: literal recipe
    eps = np.random.Generator(np.random.PCG64(np.random.SeedSequence([5, 9]))).standard_normal((3, 2, 16))
    np.testing.assert_allclose(rows, (0.8 * q.astype(np.float64)[None] + 0.6 * eps).astype(np.float32), rtol=0, atol=0)
