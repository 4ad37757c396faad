"""Jensen-bias correction of cached-key scores.

Source: the abstract (a per-score correction, removing the bias in expectation,
computed on the fly from the cached keys' quantization step sizes and the query
norm, via a second-order Taylor approximation, with no extra memory) and the
Fig. 3 caption in §1 (zero-mean uniform quantization noise delta on a score;
E[e^(s+delta)] exceeds e^s by convexity of exp; subtracting b moves E[e^(s_hat-b)]
back toward e^s). The derivation section itself (§4) is not among the pages, so
the correction is derived here from that model; this is the plainest reading
and it is listed in the design notes.

Derivation. A cached key k is stored as k_hat = k + eps in the rotated basis
(Eq. (1)), with eps_c independent and uniform on [-Delta_c/2, Delta_c/2]
(the classical uniform model of rounding noise). The scaled score of query q
(rotated q' = H q, softmax scale s) is s q'.k_hat = s q'.k + sum_c s q'_c eps_c.
For u uniform on [-D/2, D/2], E[exp(a u)] = sinh(a D/2) / (a D/2). With
x_c = s q'_c Delta_c / 2 the score's exponential is inflated by the factor
prod_c sinh(x_c)/x_c, so the exact correction is

    b_exact = sum_c log(sinh(x_c) / x_c) >= 0,

and since log(sinh(x)/x) = x^2/6 - x^4/180 + x^6/2835 - ..., its second-order
Taylor form is

    b = sum_c x_c^2 / 6 = s^2 sum_c q'_c^2 Delta_c^2 / 24,

which for one step per token (Delta_c = Delta_j) is s^2 ||q||^2 Delta_j^2 / 24
(||q'|| = ||q||): the query norm and the key's step size, as the abstract says.
The correction applies to cached (quantized) keys only; current-chunk keys are
unquantized and get none (abstract; §1).
"""
from __future__ import annotations

import numpy as np


def log_sinhc(x: np.ndarray) -> np.ndarray:
    """phi(x) = log(sinh(x)/x), even in x, computed without cancellation (float64)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    out = np.empty_like(a)
    small = a < 1e-2
    s2 = a[small] ** 2
    out[small] = s2 / 6.0 - s2 ** 2 / 180.0 + s2 ** 3 / 2835.0
    big = ~small
    ab = a[big]
    # sinh(a)/a = e^a (1 - e^{-2a}) / (2a)
    out[big] = ab + np.log(-np.expm1(-2.0 * ab)) - np.log(2.0 * ab)
    return out


def bias_taylor_per_token(q_rot: np.ndarray, delta_tok: np.ndarray, s: float) -> np.ndarray:
    """b_ij = s^2 ||q'_i||^2 Delta_j^2 / 24 ; q_rot [nq, d], delta_tok [nk] -> [nq, nk]."""
    qn2 = np.sum(np.asarray(q_rot, dtype=np.float64) ** 2, axis=-1)
    return (s * s / 24.0) * qn2[:, None] * (np.asarray(delta_tok, dtype=np.float64) ** 2)[None, :]


def bias_taylor_per_channel(q_rot: np.ndarray, delta_ch: np.ndarray, s: float) -> np.ndarray:
    """b_ij = s^2 sum_c q'_ic^2 Delta_jc^2 / 24 ; delta_ch [nk, d] -> [nq, nk]."""
    q2 = np.asarray(q_rot, dtype=np.float64) ** 2
    d2 = np.asarray(delta_ch, dtype=np.float64) ** 2
    return (s * s / 24.0) * (q2 @ d2.T)


def bias_exact(q_rot: np.ndarray, delta: np.ndarray, s: float) -> np.ndarray:
    """b_ij = sum_c log(sinh(x)/x), x = s q'_ic Delta_jc / 2.

    ``delta`` is per token [nk] or per channel [nk, d]. Cost is nq*nk*d
    transcendental evaluations: meant for small shapes and sampled rows.
    """
    q = np.asarray(q_rot, dtype=np.float64)
    dl = np.asarray(delta, dtype=np.float64)
    if dl.ndim == 1:
        dl = np.repeat(dl[:, None], q.shape[1], axis=1)
    out = np.empty((q.shape[0], dl.shape[0]))
    for i in range(q.shape[0]):
        x = 0.5 * s * q[i][None, :] * dl
        out[i] = log_sinhc(x).sum(axis=1)
    return out
