"""The seeded generator: native fills equal the numpy statement of the definition,
slices are reproducible on their own, and the draws have the stated moments."""
import numpy as np
import pytest

from gpt_pre_norm_amd import synth


def test_native_matches_definition():
    if synth._native() is None:
        pytest.skip("libgpt2synth.so not built")
    for start, n in ((0, 1), (1, 1), (3, 10), (12345, 4097)):
        a = synth.normal((n,), 0.02, 7, 3, start=start)
        b = synth.normal((n,), 0.02, 7, 3, start=start, native=False)
        assert np.array_equal(a, b)
    assert np.array_equal(synth.token_ids((999,), 50257, 3, 2),
                          synth.token_ids((999,), 50257, 3, 2, native=False))


def test_slices_are_independent_of_the_rest():
    full = synth.normal((1000,), 1.0, 5, 9)
    assert np.array_equal(full[333:777], synth.normal((444,), 1.0, 5, 9, start=333))
    bits = synth.normal_bf16_bits((1000,), 1.0, 5, 9)
    assert np.array_equal(synth.bf16_bits_to_f32(bits), synth.round_bf16(full))


def test_moments_and_ranges():
    x = synth.normal((1 << 20,), 1.0, 1, 1)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1) < 5e-3
    ids = synth.token_ids((1 << 16,), 50257, 1, 2)
    assert ids.min() >= 0 and ids.max() < 50257


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-3], np.float32)
    r = synth.round_bf16(f)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1.0 + 2 ** -6 and r[3] == -2.5
    assert abs(r[4] - 3.0e-3) <= 2 ** -8 * 3.0e-3
