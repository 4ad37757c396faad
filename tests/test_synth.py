"""The seeded generator: deterministic, slice-consistent, with the stated shapes and outliers."""
import numpy as np

from bit_kv_cache_kvq_amd import synth


def test_deterministic_and_slice_consistent():
    w = synth.WORKLOADS["tiny"]
    a = synth.draw_all(w)
    b = synth.draw_all(w)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    one = synth.draw(w, "k_cache", heads=[(0, 1)])
    np.testing.assert_array_equal(one[0], a["k_cache"][0, 1])
    assert a["q"].shape == (1, 2, 128, 64) and a["k_cache"].shape == (1, 2, 256, 64)
    assert a["q"].dtype == np.uint16


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], dtype=np.float32)
    r = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    np.testing.assert_array_equal(r, [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0])


def test_outlier_channels_and_t3():
    w = synth.WORKLOADS["c24"]
    k = synth.bf16_bits_to_f32(synth.draw(w, "k_cache", heads=[(0, 0)])[0])
    std = k.std(axis=0)
    assert np.all(std[:4] > 8) and np.all(std[4:] < 1.2)
    w4 = synth.WORKLOADS["c40_perch"]
    k4 = synth.bf16_bits_to_f32(synth.draw(w4, "k_cur", heads=[(0, 0)])[0])
    # Student-t(3): heavy tails, variance 3
    assert np.abs(k4).max() > 15 and 2.0 < k4.var() < 5.0
