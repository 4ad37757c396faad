"""Pins of the Jensen-bias correction (abstract; Fig. 3 caption in §1).

The correction is derived from the uniform rounding-noise model of Fig. 3; these
tests pin the derivation against quadrature, Monte Carlo sampling of that
model, the Taylor series of log(sinh x / x) and its special cases.
"""
import numpy as np
import pytest
from scipy import integrate

from oracle.correction import bias_exact, bias_taylor_per_channel, bias_taylor_per_token, log_sinhc


@pytest.mark.parametrize("a,delta", [(0.3, 0.5), (1.0, 1.0), (2.5, 1.7), (-4.0, 2.0), (10.0, 1.5), (1e-3, 0.2)])
def test_uniform_noise_closed_form_by_quadrature(a, delta):
    # E[exp(a u)], u ~ U[-delta/2, delta/2], by numerical integration
    val, _ = integrate.quad(lambda u: np.exp(a * u) / delta, -delta / 2, delta / 2, epsabs=0, epsrel=1e-13)
    np.testing.assert_allclose(log_sinhc(a * delta / 2), np.log(val), rtol=1e-9, atol=1e-15)


def test_taylor_coefficients():
    # log(sinh x / x) = x^2/6 - x^4/180 + ... : second order is x^2/6, i.e. a^2 Delta^2 / 24
    for x in [1e-4, 1e-3, 1e-2, 0.05]:
        assert abs(log_sinhc(x) / (x * x / 6) - 1) < x * x / 30 + 1e-12
    x = np.linspace(-1, 1, 2001)
    gap = x ** 2 / 6 - log_sinhc(x)
    assert np.all(gap >= -1e-15)
    assert np.all(gap <= x ** 4 / 180 + 1e-15)
    # fourth-order coefficient
    x = 0.01
    np.testing.assert_allclose((x * x / 6 - log_sinhc(x)) / x ** 4, 1 / 180, rtol=1e-3)


def test_exact_bias_nonnegative_and_zero_cases():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((5, 16))
    dl = rng.uniform(0, 2, 7)
    s = 0.25
    b = bias_exact(q, dl, s)
    assert np.all(b >= 0)                            # Jensen: the inflation factor is >= 1
    np.testing.assert_array_equal(bias_exact(q, np.zeros(7), s), 0)
    np.testing.assert_array_equal(bias_exact(np.zeros((5, 16)), dl, s), 0)
    np.testing.assert_array_equal(bias_taylor_per_token(q, np.zeros(7), s), 0)


def test_taylor_scaling_and_sandwich():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((6, 32))
    dl = rng.uniform(0.1, 1.0, 9)
    s = 1 / np.sqrt(32)
    b = bias_taylor_per_token(q, dl, s)
    np.testing.assert_allclose(bias_taylor_per_token(2 * q, dl, s), 4 * b, rtol=1e-14)
    np.testing.assert_allclose(bias_taylor_per_token(q, 3 * dl, s), 9 * b, rtol=1e-14)
    be = bias_exact(q, dl, s)
    x = 0.5 * s * q[:, None, :] * dl[None, :, None]
    assert np.all(np.abs(x) <= 1)
    assert np.all(b - be >= -1e-15)
    assert np.all(b - be <= (x ** 4 / 180).sum(-1) + 1e-15)


def test_per_channel_reduces_to_per_token():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((4, 64))
    dl = rng.uniform(0.1, 2, 5)
    np.testing.assert_allclose(bias_taylor_per_channel(q, np.repeat(dl[:, None], 64, 1), 0.3),
                               bias_taylor_per_token(q, dl, 0.3), rtol=1e-14)
    np.testing.assert_allclose(bias_exact(q, np.repeat(dl[:, None], 64, 1), 0.3), bias_exact(q, dl, 0.3),
                               rtol=1e-14)


@pytest.mark.parametrize("d", [4, 16])
def test_monte_carlo_jensen_gap(d):
    # sample the noise model directly: log E[exp(s q.eps)] with eps_c ~ U[-D_c/2, D_c/2]
    rng = np.random.default_rng(12 + d)
    q = rng.standard_normal(d)
    dl = rng.uniform(0.2, 1.5, d)
    s = 1 / np.sqrt(d)
    n = 1_000_000
    eps = (rng.random((n, d)) - 0.5) * dl
    e = np.exp(s * eps @ q)
    mean, se = e.mean(), e.std() / np.sqrt(n)
    gap = np.log(mean)
    be = bias_exact(q[None], dl[None, :], s)[0, 0]
    bt = bias_taylor_per_channel(q[None], dl[None, :], s)[0, 0]
    assert abs(gap - be) <= 4 * se / mean
    # subtracting b moves E[e^(s_hat - b)] back to e^s: exactly for b_exact, closely for Taylor
    assert abs(mean * np.exp(-be) - 1) <= 4 * se / mean
    assert abs(mean * np.exp(-bt) - 1) < abs(mean - 1)
    # the Taylor term sits above the sampled gap by at most the fourth-order remainder
    x = 0.5 * s * q * dl
    rem = (x ** 4 / 180).sum()
    assert -4 * se / mean <= bt - gap <= rem + 4 * se / mean
    assert gap > 0


def test_per_channel_bias_uses_rotated_query_monte_carlo():
    # Per-channel steps live in the rotated basis: the stored-basis error eps (uniform per
    # channel) perturbs the un-rotated key by H eps, so the score noise is s q.(H eps) =
    # s (Hq).eps. Sample that directly and compare with the oracle's bias for rotated
    # per-channel keys, which must use the rotated query.
    from oracle.attention import _bias_fn
    from oracle.hadamard import sylvester
    from oracle.quant import Format
    rng = np.random.default_rng(40)
    d, group = 16, 64
    H = sylvester(d)
    q = rng.standard_normal((1, d)) * 2
    delta = np.zeros((1, 1, 1, d), dtype=np.float16)
    delta[0, 0, 0] = rng.uniform(0.05, 1.5, d).astype(np.float16)
    cache = {"k_scale": delta, "n_chunks": 1}
    fmt = Format(2, "channel", group, True, "key")
    s = 1 / np.sqrt(d)
    b = _bias_fn(q, cache, 0, 0, group, fmt, s, "exact")(np.array([0]))[0, 0]
    dl = delta[0, 0, 0].astype(np.float64)
    n = 1_000_000
    eps = (rng.random((n, d)) - 0.5) * dl
    e = np.exp(s * (eps @ H) @ q[0])
    mean, se = e.mean(), e.std() / np.sqrt(n)
    assert abs(np.log(mean) - b) <= 4 * se / mean
    b_unrot = bias_exact(q, dl[None, :], s)[0, 0]
    assert abs(np.log(mean) - b_unrot) > 8 * se / mean   # the rotation matters for this q
