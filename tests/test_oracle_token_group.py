"""Pins of the oracle's group-wise per-token granularity (paper §3, "Quantization granularity":
each token's d channels split into groups of g, each group with its own (Delta, z)).

What pins it from outside the code under test:
* g = d is per-token quantization (already pinned by worked examples and brute force);
* every (token, group) pair equals a plain per-vector quantization of that group's rotated
  channels, found by explicit loops;
* reconstruction error is at most half of the group's own step (Eq. (1));
* the correction for group-wise keys equals the per-group sum
  s^2 sum_groups ||q'_grp||^2 Delta_grp^2 / 24 written out by loops, and reduces to the
  per-token form when all groups of a key share one step;
* corrected attention mass moves toward the BF16 mass (Fig. 2) with group-wise keys too.
"""
import numpy as np
import pytest

import oracle
from bit_kv_cache_kvq_amd import synth
from oracle.correction import bias_taylor_per_token
from oracle.hadamard import fwht_f32
from oracle.quant import (Format, bf16_to_f32, chunk_pad, dequant_window, pack_window, quantize_chunk,
                          quantize_lastaxis, step_token_group_key)


def _x(shape, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    x[..., 3] *= 10.0
    return synth.f32_to_bf16_bits(x)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("role", ["key", "value"])
def test_group_of_d_channels_is_per_token(bits, role):
    x = _x((1, 2, 200, 64), 1)
    tok = pack_window(x, 100, Format(bits, "token", 128, True, role))
    grp = pack_window(x, 100, Format(bits, "token_group", 64, True, role))
    np.testing.assert_array_equal(tok[0], grp[0])
    np.testing.assert_array_equal(tok[1], grp[1][..., 0])
    np.testing.assert_array_equal(tok[2], grp[2][..., 0])


@pytest.mark.parametrize("g", [16, 32, 64])
def test_each_group_is_its_own_vector(g):
    x = _x((1, 1, 9, 128), 2)
    codes, delta, z = quantize_chunk(x, Format(2, "token_group", g, True, "key"))
    y = fwht_f32(bf16_to_f32(x))
    for t in range(9):
        for j in range(128 // g):
            cj, dj, zj = quantize_lastaxis(y[0, 0, t, j * g:(j + 1) * g][None], 2)
            np.testing.assert_array_equal(codes[0, 0, t, j * g:(j + 1) * g], cj[0])
            assert delta[0, 0, t, j] == dj[0] and z[0, 0, t, j] == zj[0]
            # the step covers that group's own range, not the token's
            seg = y[0, 0, t, j * g:(j + 1) * g]
            assert dj[0] == np.float32(np.float16((seg.max() - seg.min()) / np.float32(3)))


@pytest.mark.parametrize("role", ["key", "value"])
def test_dequant_error_within_half_group_step(role):
    x = _x((1, 2, 130, 128), 3)
    fmt = Format(2, "token_group", 32, False, role)
    words, scale, zero = pack_window(x, 65, fmt)
    cp = chunk_pad(65)
    assert scale.shape == (1, 2, 2 * cp, 4) and zero.shape == scale.shape
    assert not scale[:, :, 65:cp].any() and not scale[:, :, cp + 65:].any()  # pad tokens
    xh = dequant_window(words, scale, zero, 65, 2, fmt)
    step = step_token_group_key(scale, 65, 2, 32)
    err = np.abs(xh - bf16_to_f32(x).astype(np.float64))
    # rounding to the grid: at most half a step (the fp16 step may round the range down by
    # 2^-11 relative, which can push the extreme value past the grid by that much)
    assert (err <= step * (0.5 + 3 * 2.0 ** -11) + 1e-12).all()


def test_group_wise_bias_is_sum_over_groups():
    rng = np.random.default_rng(5)
    x = _x((1, 1, 64, 128), 6)
    fmt = Format(2, "token_group", 32, True, "key")
    _, scale, _ = pack_window(x, 64, fmt)
    q = rng.standard_normal((5, 128))
    s = 1 / np.sqrt(128)
    qrot = oracle.hadamard.rotate_f64(q)
    delta = step_token_group_key(scale, 64, 1, 32)[0, 0]
    b = oracle.correction.bias_taylor_per_channel(qrot, delta, s)
    for i in range(5):
        for j in range(64):
            ref = 0.0
            for grp in range(4):
                n2 = sum(qrot[i, c] ** 2 for c in range(32 * grp, 32 * grp + 32))
                ref += s * s * n2 * float(scale[0, 0, j, grp]) ** 2 / 24
            assert abs(b[i, j] - ref) <= 1e-12 * max(1.0, ref)
    # equal steps within each key: the per-token form s^2 ||q||^2 Delta_j^2 / 24
    flat = np.repeat(delta[:, :1], 128, axis=1)
    np.testing.assert_allclose(oracle.correction.bias_taylor_per_channel(qrot, flat, s),
                               bias_taylor_per_token(q, delta[:, 0], s), rtol=1e-12)


def test_attention_group_of_d_equals_per_token():
    w = synth.WORKLOADS["tiny"]
    x = synth.draw_all(w)
    args = (x["q"], x["k_cache"], x["v_cache"], x["k_cur"], x["v_cur"])
    kw = dict(chunk_len=w.chunk_len, correction="taylor")
    O1, P1, _, _ = oracle.reference_call(*args, k_fmt=Format(2, "token", 128, True, "key"),
                                         v_fmt=Format(2, "token", 128, True, "value"), **kw)
    O2, P2, _, _ = oracle.reference_call(*args, k_fmt=Format(2, "token_group", w.d, True, "key"),
                                         v_fmt=Format(2, "token_group", w.d, True, "value"), **kw)
    # same dequantized window; the bias differs only in float64 summation order
    np.testing.assert_allclose(O1, O2, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(P1, P2, rtol=1e-10)


@pytest.mark.parametrize("g", [32, 64])
def test_group_wise_keys_correction_restores_mass(g):
    # Fig. 2 with group-wise keys: smaller groups give smaller steps, yet the cached-block
    # mass is still inflated by rounding noise, and the correction pulls it back.
    w = synth.WORKLOADS["c24"]
    x = synth.draw_all(w, heads=[(0, 0)])
    x = {k: v[None] for k, v in x.items()}
    kf, vf = Format(2, "token_group", g, True, "key"), Format(2, "token_group", g, True, "value")
    args = (x["q"], x["k_cache"], x["v_cache"], x["k_cur"], x["v_cur"])
    kw = dict(chunk_len=w.chunk_len, k_fmt=kf, v_fmt=vf, rows=np.arange(192))
    _, ps_b, _, _ = oracle.reference_call(*args, quantized=False, **kw)
    _, ps_u, _, cache = oracle.reference_call(*args, correction="none", **kw)
    _, ps_c, _, _ = oracle.reference_call(*args, correction="taylor", cache=cache, **kw)
    assert (ps_u - ps_b).mean() > 0
    assert np.abs(ps_c - ps_b).mean() < np.abs(ps_u - ps_b).mean()
