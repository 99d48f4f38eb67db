"""The seeded input generator: distributions, reproducibility, host/device twins."""
import numpy as np

import synth


def test_codes_uniform_and_reproducible():
    key = synth.layer_key(0, 1, 0)
    c = synth.ternary_codes(key, 0, 256, 5120)
    assert c.dtype == np.int8 and set(np.unique(c)) == {-1, 0, 1}
    n = c.size
    for v in (-1, 0, 1):
        frac = np.mean(c == v)
        assert abs(frac - 1 / 3) < 4 * np.sqrt(2 / 9 / n)
    np.testing.assert_array_equal(c, synth.ternary_codes(key, 0, 256, 5120))
    # rows are addressable on their own
    np.testing.assert_array_equal(c[100:110], synth.ternary_codes(key, 100, 10, 5120))
    # different layers differ
    assert np.mean(c == synth.ternary_codes(synth.layer_key(0, 1, 1), 0, 256, 5120)) < 0.4


def test_codes_torch_twin_matches_numpy():
    import torch
    key = synth.layer_key(0, 4, 77)
    a = synth.ternary_codes(key, 5, 33, 1024)
    b = synth.ternary_codes_torch(key, 5, 33, 1024, "cpu")
    assert b.dtype == torch.int8
    np.testing.assert_array_equal(a, b.numpy())


def test_scales_lognormal():
    s = synth.group_scales(0, 1, 0, 1024, 5120).astype(np.float64)
    ls = np.log(s)
    assert abs(ls.mean() + 4.0) < 0.01 and abs(ls.std() - 0.5) < 0.01
    assert np.all(np.isfinite(s)) and np.all(s > 0)


def test_activations_outliers_and_range():
    K = 5120
    bits = synth.activations(0, 1, 0, 16, K)
    x = synth.bf16_bits_to_f32(bits).astype(np.float64)
    chans = synth.outlier_channels(0, 1, 0, K)
    assert len(chans) == 26
    big = np.abs(x).mean(axis=0)
    assert np.all(big[chans] > 5.0)
    mask = np.ones(K, bool)
    mask[chans] = False
    assert abs(np.std(x[:, mask]) - 1.0) < 0.05
    nz = x[x != 0]
    assert np.all(np.abs(nz) >= 2.0 ** -24) and np.all(np.abs(x) < 256)
    # every value is a multiple of 2**-31 (bf16 with the small values flushed)
    assert np.all(np.ldexp(x, 31) == np.rint(np.ldexp(x, 31)))
    # the first b tokens of a larger draw are the b-token draw
    np.testing.assert_array_equal(synth.activations(0, 1, 0, 4, K), bits[:4])


def test_bf16_rounding_ties_even():
    v = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5], dtype=np.float32)
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(v))
    np.testing.assert_array_equal(got, np.array([1.0, 1 + 2 ** -6, -2.5], dtype=np.float32))
