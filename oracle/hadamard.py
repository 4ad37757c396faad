"""Hadamard rotation (paper §3 "Hadamard rotation").

The paper rotates keys (and queries) by an orthogonal Hadamard matrix H with
H^T H = I before quantizing, which spreads channel outliers over all channels
while leaving every score unchanged, because (Hq)^T (Hk) = q^T k. The rotation
is built on the normalized Sylvester matrix of order d (a power of two),
H[i][j] = (-1)^popcount(i & j) / sqrt(d), which is symmetric and its own
inverse. §3 names a randomized Hadamard rotation (QuaRot's): R = H diag(s) with
a fixed sign vector s in {+1, -1}^d, so x' = R x flips the signs of the
channels with s_c = -1 and then applies H; R^T R = I, (R q)^T (R k) = q^T k,
and R^{-1} = R^T = diag(s) H. Without a sign vector (s = 1) R is H itself.
"""
from __future__ import annotations

import numpy as np


def sylvester(d: int) -> np.ndarray:
    """Normalized Sylvester-Hadamard matrix of order d in float64, by Kronecker products."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    base = np.array([[1.0, 1.0], [1.0, -1.0]])
    while h.shape[0] < d:
        h = np.kron(h, base)
    return h / np.sqrt(d)


def sign_vector(signs, d: int) -> np.ndarray:
    """The diagonal s of diag(s) as float64 [d]: all +1 for an empty ``signs``."""
    if signs is None or len(signs) == 0:
        return np.ones(d)
    s = np.asarray(signs, dtype=np.float64)
    if s.shape != (d,) or not np.all(np.abs(s) == 1):
        raise ValueError("signs must hold d values of +1 or -1")
    return s


def rotate_f64(x: np.ndarray, signs=()) -> np.ndarray:
    """y = H_d diag(s) x for every vector along the last axis, in float64 (a plain matmul)."""
    d = x.shape[-1]
    return (np.asarray(x, dtype=np.float64) * sign_vector(signs, d)) @ sylvester(d)  # H is symmetric


def unrotate_f64(y: np.ndarray, signs=()) -> np.ndarray:
    """x = diag(s) H_d y, the inverse of ``rotate_f64``, in float64."""
    d = y.shape[-1]
    return (np.asarray(y, dtype=np.float64) @ sylvester(d)) * sign_vector(signs, d)


def flip_f32(x: np.ndarray, signs=()) -> np.ndarray:
    """diag(s) x in float32: an exact negation of the channels with s_c = -1 (the first
    step of the randomized transform; the float32 butterflies follow)."""
    x = np.asarray(x, dtype=np.float32)
    if signs is None or len(signs) == 0:
        return x
    return x * sign_vector(signs, x.shape[-1]).astype(np.float32)


def scale_f32(d: int) -> np.float32:
    """The float32 nearest to 1/sqrt(d): the normalizing factor of the float32 transform."""
    return np.float32(1.0 / np.sqrt(np.float64(d)))


def fwht_f32(x: np.ndarray) -> np.ndarray:
    """H_d x in float32 with one fixed operation order (the quantizer's contract).

    Butterfly stages run for h = 1, 2, 4, ..., d/2 in that order. In stage h,
    every index i with bit h clear is paired with i + h and the pair (a, b)
    becomes (a + b, a - b), one float32 add or subtract each. After the last
    stage every element is multiplied once by ``scale_f32(d)``. The result
    depends on this order only through float32 rounding; in exact arithmetic it
    is ``sylvester(d) @ x``.
    """
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    lead = y.shape[:-1]
    h = 1
    while h < d:
        v = y.reshape(lead + (d // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        y = v.reshape(lead + (d,))
        h *= 2
    return y * scale_f32(d)
