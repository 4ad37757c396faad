"""Chunk attention over [cached window ; current chunk] with the Jensen-bias correction.

Source: abstract and §1 of the paper. In chunk-wise autoregressive video
diffusion the queries of the chunk being denoised attend to the keys and values
of a sliding window of previously generated chunks, kept in a KV cache, and to
the keys and values of their own chunk, which are not quantized. The correction
b is subtracted from the scores of cached keys before the softmax; the
cached-block and current-chunk attention masses P_S and P_R (Fig. 2 caption)
are the shares of the softmax mass that fall on each block.

Readings (listed in the design notes): no causal mask inside the current chunk (every
query sees the whole window and the whole current chunk); softmax scale
s = 1/sqrt(d); the correction is applied in the same scaled-score units the
softmax sees (``correction.py``).

Everything here is float64: for each query row
    l_ij = s q_i.k_hat_j - b_ij   (cached j),   l_ir = s q_i.k_r   (current r)
    m_i = max over both, e = exp(l - m)
    O_i  = (sum_j e_ij v_hat_j + sum_r e_ir v_r) / sum e
    P_S,i = sum_j e_ij / sum e,   P_R,i = sum_r e_ir / sum e.
Rows are independent, so they are processed in blocks; that changes no result
beyond float64 rounding.
"""
from __future__ import annotations

import numpy as np

from . import correction as corr
from .hadamard import rotate_f64
from .quant import (Format, bf16_to_f32, dequant_window, pack_window, step_per_channel_key,
                    step_per_token_key, step_token_group_key)


def attend_head(q, k_c, v_c, k_r, v_r, s, bias=None, block=256):
    """Exact attention for one head (float64). ``bias(rows) -> [len(rows), n_c]`` or None."""
    q = np.asarray(q, dtype=np.float64)
    nq, d = q.shape
    n_c, n_r = k_c.shape[0], k_r.shape[0]
    O = np.empty((nq, v_c.shape[1] if n_c else v_r.shape[1]))
    PS = np.empty(nq)
    PR = np.empty(nq)
    buf_c = np.empty((min(block, nq), n_c))
    buf_r = np.empty((min(block, nq), n_r))
    for r0 in range(0, nq, block):
        r1 = min(nq, r0 + block)
        rows = np.arange(r0, r1)
        lc = buf_c[: r1 - r0]
        lr = buf_r[: r1 - r0]
        np.matmul(q[r0:r1], k_c.T, out=lc)
        lc *= s
        if bias is not None:
            lc -= bias(rows)
        np.matmul(q[r0:r1], k_r.T, out=lr)
        lr *= s
        m = np.maximum(lc.max(axis=1, initial=-np.inf), lr.max(axis=1, initial=-np.inf))
        lc -= m[:, None]
        np.exp(lc, out=lc)
        lr -= m[:, None]
        np.exp(lr, out=lr)
        zs = lc.sum(axis=1)
        zr = lr.sum(axis=1)
        tot = zs + zr
        O[r0:r1] = (lc @ v_c + lr @ v_r) / tot[:, None]
        PS[r0:r1] = zs / tot
        PR[r0:r1] = zr / tot
    return O, PS, PR


def quantize_cache(k_cache_bits, v_cache_bits, chunk_len, k_fmt: Format, v_fmt: Format):
    """Pack the cached window with the oracle's quantizer; returns words/scales and fp64 dequants."""
    kw, ks, kz = pack_window(k_cache_bits, chunk_len, k_fmt)
    vw, vs, vz = pack_window(v_cache_bits, chunk_len, v_fmt)
    n_chunks = k_cache_bits.shape[-2] // chunk_len
    k_hat = dequant_window(kw, ks, kz, chunk_len, n_chunks, k_fmt)
    v_hat = dequant_window(vw, vs, vz, chunk_len, n_chunks, v_fmt)
    return {"k_words": kw, "k_scale": ks, "k_zero": kz, "v_words": vw, "v_scale": vs, "v_zero": vz,
            "k_hat": k_hat, "v_hat": v_hat, "n_chunks": n_chunks}


def reference_call(q_bits, k_cache_bits, v_cache_bits, k_cur_bits, v_cur_bits, *, chunk_len,
                   k_fmt: Format, v_fmt: Format, correction="taylor", softmax_scale=None,
                   rows=None, quantized=True, cache=None, block=256):
    """Oracle for one call. Inputs are bf16 bit arrays [B, H, n, d].

    correction: "none" | "taylor" | "exact". quantized=False gives the BF16
    reference: the cached window unquantized and no correction. ``rows``
    restricts the query rows (same rows for every head). ``cache`` may hold the
    result of ``quantize_cache`` to skip re-packing. Returns (O, P_S, P_R, cache)
    with O [B, H, nq, d] float64.
    """
    B, H, nq, d = q_bits.shape
    s = float(softmax_scale) if softmax_scale else 1.0 / np.sqrt(d)
    if quantized and cache is None:
        cache = quantize_cache(k_cache_bits, v_cache_bits, chunk_len, k_fmt, v_fmt)
    if rows is None:
        rows = np.arange(nq)
    rows = np.asarray(rows)
    O = np.empty((B, H, len(rows), d))
    PS = np.empty((B, H, len(rows)))
    PR = np.empty((B, H, len(rows)))
    for b in range(B):
        for h in range(H):
            q = bf16_to_f32(q_bits[b, h, rows]).astype(np.float64)
            k_r = bf16_to_f32(k_cur_bits[b, h]).astype(np.float64)
            v_r = bf16_to_f32(v_cur_bits[b, h]).astype(np.float64)
            if not quantized:
                k_c = bf16_to_f32(k_cache_bits[b, h]).astype(np.float64)
                v_c = bf16_to_f32(v_cache_bits[b, h]).astype(np.float64)
                bias = None
            else:
                k_c = cache["k_hat"][b, h]
                v_c = cache["v_hat"][b, h]
                bias = _bias_fn(q, cache, b, h, chunk_len, k_fmt, s, correction)
            O[b, h], PS[b, h], PR[b, h] = attend_head(q, k_c, v_c, k_r, v_r, s, bias, block)
    return O, PS, PR, cache


def _bias_fn(q, cache, b, h, chunk_len, k_fmt: Format, s, correction):
    if correction == "none":
        return None
    q_rot = rotate_f64(q, k_fmt.signs) if k_fmt.hadamard else q
    n_chunks = cache["n_chunks"]
    if k_fmt.granularity == "token":
        delta = step_per_token_key(cache["k_scale"][b:b + 1, h:h + 1], chunk_len, n_chunks)[0, 0]
        if correction == "taylor":
            return lambda rows: corr.bias_taylor_per_token(q_rot[rows], delta, s)
        return lambda rows: corr.bias_exact(q_rot[rows], delta, s)
    if k_fmt.granularity == "token_group":
        # a step per (key, channel): the general form b = s^2 sum_c q'_c^2 Delta_jc^2 / 24
        delta = step_token_group_key(cache["k_scale"][b:b + 1, h:h + 1], chunk_len, n_chunks, k_fmt.group)[0, 0]
    else:
        delta = step_per_channel_key(cache["k_scale"][b:b + 1, h:h + 1], chunk_len, n_chunks, k_fmt.group)[0, 0]
    if correction == "taylor":
        return lambda rows: corr.bias_taylor_per_channel(q_rot[rows], delta, s)
    return lambda rows: corr.bias_exact(q_rot[rows], delta, s)
