"""Asymmetric round-to-nearest quantization of KV-cache chunks (paper §3).

Eq. (1) of §3 maps a value x to the code
    x_q = clamp(round(x / Delta) + z, 0, 2^B - 1)
and reconstructs x_hat = (x_q - z) * Delta, with |x_hat - x| <= Delta / 2 when
Delta and z are chosen to cover the group's whole [min, max] range. §3
"Quantization granularity" lets one (Delta, z) pair be shared per token, per
group of channels of a token, or per tensor; keys may also share one pair per
channel over a group of tokens (the KIVI-style per-channel key scheme named in
§2). The paper quantizes keys and values after a Hadamard rotation (Fig. 1
caption: asymmetric INT2 with the QuaRot rotation and round-to-nearest, on keys and
values).

Readings where the pages leave a step open (each is also listed in the design notes):

* Delta = (max - min) / (2^B - 1), stored as fp16 (round to nearest even);
  z = round(-min / Delta), an integer, not clamped to [0, 2^B - 1], stored as
  fp16 (exact for |z| <= 2048). "round" is round-half-to-even.
* A group with Delta == 0 after fp16 rounding stores Delta = z = +0 and codes 0.
* z = -0 is canonicalized to +0.
* The codes, Delta and z are integers or fp16 values decided by floating point,
  so this module fixes one float32 operation order (below); the kernel follows
  the same order, which is what makes bit-exact comparison meaningful.

float32 operation order for one group G (values y, already rotated):
  1. mn = min(y), mx = max(y)
  2. d32 = (mx - mn) / float32(2^B - 1)            correctly rounded division
  3. delta = float32(fp16_rne(d32))
  4. if delta == 0: scale = zero = +0, codes = 0
  5. z = rint(-mn / delta) + 0.0                      rint = half-to-even
  6. code = min(max(rint(y / delta) + z, 0), 2^B - 1)
  7. scale = fp16(delta), zero = fp16(z)

Storage layouts (the library's documented format, restated here independently):

* Tokens of each cached chunk are padded to a multiple of 64 (``chunk_pad``);
  pad tokens hold code 0, and per-token scale and zero 0.
* Keys, token-major: with c = 32 / B codes per 32-bit word, word w of a token
  holds channels c*w .. c*w + c - 1, channel c*w + i in bits [B*i, B*i + B).
  Window array shape [B, H, n_chunks * chunk_pad, d / c].
* Values, 64-token channel-major blocks: block t holds tokens 64t .. 64t + 63
  of the padded token axis; inside it, channel ch has 64 / c words and word u
  holds tokens c*u .. c*u + c - 1, token c*u + i in bits [B*i, B*i + B).
  Window array shape [B, H, n_chunks * chunk_pad / 64, d, 64 / c].
* Per-token scale and zero: fp16 [B, H, n_chunks * chunk_pad].
  Group-wise per token (§3's third granularity: each token's d channels split into
  groups of g = ``group`` channels, group j holding its own (Delta_ij, z_ij)):
  fp16 [B, H, n_chunks * chunk_pad, d / g], pad tokens 0.
  Per-channel (keys only): fp16 [B, H, n_chunks * ceil(chunk_len / group), d];
  groups restart at each chunk's first token.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .hadamard import flip_f32, fwht_f32, unrotate_f64

TOKEN_BLOCK = 64


@dataclasses.dataclass(frozen=True)
class Format:
    bits: int = 2                 # 2 or 4
    granularity: str = "token"    # "token" | "token_group" | "channel" (channel: keys only)
    group: int = 128              # channel: tokens per channel group; token_group: channels per group
    hadamard: bool = True
    role: str = "key"             # "key" (token-major words) | "value" (channel-major blocks)
    signs: tuple = ()             # randomized rotation H diag(s): d values of +1/-1; () is s = 1


def chunk_pad(chunk_len: int) -> int:
    return -(-chunk_len // TOKEN_BLOCK) * TOKEN_BLOCK


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize_lastaxis(y: np.ndarray, bits: int):
    """The float32 contract above, with one group per vector along the last axis.

    Returns (codes uint8, delta float32, z float32); delta and z are the values
    whose fp16 images are stored (both are exact in fp16 by construction,
    z up to |z| <= 2048).
    """
    y = np.asarray(y, dtype=np.float32)
    qmax = np.float32(2 ** bits - 1)
    mn = y.min(axis=-1)
    mx = y.max(axis=-1)
    d32 = (mx - mn) / qmax
    delta = d32.astype(np.float16).astype(np.float32)
    ok = delta != 0
    safe = np.where(ok, delta, np.float32(1.0))
    z = np.rint(-mn / safe) + np.float32(0.0)
    z = np.where(ok, z, np.float32(0.0)).astype(np.float32)
    c = np.rint(y / safe[..., None]) + z[..., None]
    c = np.minimum(np.maximum(c, np.float32(0.0)), qmax)
    c = np.where(ok[..., None], c, np.float32(0.0))
    delta = np.where(ok, delta, np.float32(0.0)).astype(np.float32)
    return c.astype(np.uint8), delta, z


def quantize_chunk(x_bits: np.ndarray, fmt: Format):
    """Quantize one chunk x [B, H, n, d] (bf16 bits) -> codes [B,H,n,d], scale, zero.

    Per-token: scale, zero are [B, H, n]. Group-wise per token: [B, H, n, d/group],
    group j of a token covering channels [j*group, (j+1)*group) of the stored basis.
    Per-channel: [B, H, ceil(n/group), d], group g covering tokens
    [g*group, min(n, (g+1)*group)).
    """
    x = bf16_to_f32(x_bits)
    if fmt.signs and not fmt.hadamard:
        raise ValueError("a sign vector needs the Hadamard rotation")
    y = fwht_f32(flip_f32(x, fmt.signs)) if fmt.hadamard else x
    B, H, n, d = y.shape
    if fmt.granularity == "token":
        codes, delta, z = quantize_lastaxis(y, fmt.bits)
        return codes, delta, z
    if fmt.granularity == "token_group":
        if d % fmt.group:
            raise ValueError("channel group does not divide d")
        codes, delta, z = quantize_lastaxis(y.reshape(B, H, n, d // fmt.group, fmt.group), fmt.bits)
        return codes.reshape(B, H, n, d), delta, z
    if fmt.granularity != "channel":
        raise ValueError(fmt.granularity)
    G = -(-n // fmt.group)
    codes = np.empty((B, H, n, d), dtype=np.uint8)
    delta = np.empty((B, H, G, d), dtype=np.float32)
    z = np.empty((B, H, G, d), dtype=np.float32)
    for g in range(G):
        t0, t1 = g * fmt.group, min(n, (g + 1) * fmt.group)
        yg = np.swapaxes(y[:, :, t0:t1, :], -1, -2)          # [B,H,d,m]
        cg, dg, zg = quantize_lastaxis(yg, fmt.bits)
        codes[:, :, t0:t1, :] = np.swapaxes(cg, -1, -2)
        delta[:, :, g, :] = dg
        z[:, :, g, :] = zg
    return codes, delta, z


def pack_key_words(codes: np.ndarray, bits: int) -> np.ndarray:
    """Token-major words: channel c*w + i of a token at bits [B*i, B*i+B) of word w."""
    cpw = 32 // bits
    *lead, n, d = codes.shape
    c = codes.astype(np.uint32).reshape(*lead, n, d // cpw, cpw)
    shifts = (np.arange(cpw, dtype=np.uint32) * np.uint32(bits))
    return np.bitwise_or.reduce(c << shifts, axis=-1).astype(np.uint32)


def unpack_key_words(words: np.ndarray, bits: int) -> np.ndarray:
    cpw = 32 // bits
    *lead, n, nw = words.shape
    shifts = (np.arange(cpw, dtype=np.uint32) * np.uint32(bits))
    c = (words[..., None] >> shifts) & np.uint32(2 ** bits - 1)
    return c.reshape(*lead, n, nw * cpw).astype(np.uint8)


def pack_value_words(codes: np.ndarray, bits: int) -> np.ndarray:
    """64-token channel-major blocks: token c*u + i of a block at bits [B*i, B*i+B) of word u."""
    cpw = 32 // bits
    *lead, n, d = codes.shape
    assert n % TOKEN_BLOCK == 0
    nb = n // TOKEN_BLOCK
    c = codes.astype(np.uint32).reshape(*lead, nb, TOKEN_BLOCK, d)
    c = np.swapaxes(c, -1, -2)                                   # [.., nb, d, 64]
    c = c.reshape(*lead, nb, d, TOKEN_BLOCK // cpw, cpw)
    shifts = (np.arange(cpw, dtype=np.uint32) * np.uint32(bits))
    return np.bitwise_or.reduce(c << shifts, axis=-1).astype(np.uint32)


def unpack_value_words(words: np.ndarray, bits: int) -> np.ndarray:
    cpw = 32 // bits
    *lead, nb, d, nw = words.shape
    shifts = (np.arange(cpw, dtype=np.uint32) * np.uint32(bits))
    c = (words[..., None] >> shifts) & np.uint32(2 ** bits - 1)   # [.., nb, d, nw, cpw]
    c = c.reshape(*lead, nb, d, nw * cpw)
    c = np.swapaxes(c, -1, -2)
    return c.reshape(*lead, nb * nw * cpw, d).astype(np.uint8)


def pack_window(x_bits: np.ndarray, chunk_len: int, fmt: Format):
    """Quantize and lay out a window of whole chunks x [B, H, n_chunks*chunk_len, d].

    Returns (words uint32, scale fp16, zero fp16) in the storage layouts above.
    """
    B, H, n, d = x_bits.shape
    if n % chunk_len:
        raise ValueError("window is not a whole number of chunks")
    nch = n // chunk_len
    cp = chunk_pad(chunk_len)
    codes_pad = np.zeros((B, H, nch * cp, d), dtype=np.uint8)
    if fmt.granularity == "token":
        scale = np.zeros((B, H, nch * cp), dtype=np.float16)
        zero = np.zeros((B, H, nch * cp), dtype=np.float16)
    elif fmt.granularity == "token_group":
        scale = np.zeros((B, H, nch * cp, d // fmt.group), dtype=np.float16)
        zero = np.zeros((B, H, nch * cp, d // fmt.group), dtype=np.float16)
    else:
        G = -(-chunk_len // fmt.group)
        scale = np.zeros((B, H, nch * G, d), dtype=np.float16)
        zero = np.zeros((B, H, nch * G, d), dtype=np.float16)
    for ci in range(nch):
        codes, delta, z = quantize_chunk(x_bits[:, :, ci * chunk_len:(ci + 1) * chunk_len, :], fmt)
        codes_pad[:, :, ci * cp: ci * cp + chunk_len, :] = codes
        if fmt.granularity in ("token", "token_group"):
            scale[:, :, ci * cp: ci * cp + chunk_len] = delta.astype(np.float16)
            zero[:, :, ci * cp: ci * cp + chunk_len] = z.astype(np.float16)
        else:
            G = delta.shape[2]
            scale[:, :, ci * G:(ci + 1) * G, :] = delta.astype(np.float16)
            zero[:, :, ci * G:(ci + 1) * G, :] = z.astype(np.float16)
    if fmt.role == "key":
        words = pack_key_words(codes_pad, fmt.bits)
    else:
        words = pack_value_words(codes_pad, fmt.bits)
    return words, scale, zero


def dequant_window(words, scale, zero, chunk_len: int, n_chunks: int, fmt: Format) -> np.ndarray:
    """Float64 reconstruction of the valid tokens of a window, in the original (un-rotated) basis.

    x_hat' = (code - z) * Delta in the stored basis (Eq. (1)), then x_hat = diag(s) H x_hat'
    when the window was rotated (the inverse of the rotation H diag(s)).
    """
    codes = unpack_key_words(words, fmt.bits) if fmt.role == "key" else unpack_value_words(words, fmt.bits)
    B, H, npad, d = codes.shape
    cp = chunk_pad(chunk_len)
    assert npad == n_chunks * cp
    out = np.empty((B, H, n_chunks * chunk_len, d), dtype=np.float64)
    for ci in range(n_chunks):
        c = codes[:, :, ci * cp: ci * cp + chunk_len, :].astype(np.float64)
        if fmt.granularity == "token":
            dl = scale[:, :, ci * cp: ci * cp + chunk_len].astype(np.float64)[..., None]
            zz = zero[:, :, ci * cp: ci * cp + chunk_len].astype(np.float64)[..., None]
        elif fmt.granularity == "token_group":
            # channel c of a token takes its group's pair (c // g)
            dl = np.repeat(scale[:, :, ci * cp: ci * cp + chunk_len].astype(np.float64), fmt.group, axis=-1)
            zz = np.repeat(zero[:, :, ci * cp: ci * cp + chunk_len].astype(np.float64), fmt.group, axis=-1)
        else:
            G = -(-chunk_len // fmt.group)
            tok_group = np.arange(chunk_len) // fmt.group
            dl = scale[:, :, ci * G:(ci + 1) * G, :].astype(np.float64)[:, :, tok_group, :]
            zz = zero[:, :, ci * G:(ci + 1) * G, :].astype(np.float64)[:, :, tok_group, :]
        out[:, :, ci * chunk_len:(ci + 1) * chunk_len, :] = (c - zz) * dl
    return unrotate_f64(out, fmt.signs) if fmt.hadamard else out


def step_per_token_key(scale, chunk_len: int, n_chunks: int) -> np.ndarray:
    """Per-token key step Delta_j (float64) of the valid tokens, [B, H, n_c]."""
    cp = chunk_pad(chunk_len)
    s = scale.astype(np.float64).reshape(scale.shape[0], scale.shape[1], n_chunks, cp)[..., :chunk_len]
    return s.reshape(scale.shape[0], scale.shape[1], n_chunks * chunk_len)


def step_token_group_key(scale, chunk_len: int, n_chunks: int, group: int) -> np.ndarray:
    """Group-wise per-token key steps expanded to channels: Delta_{j,c} = Delta_{j, c // g}
    (float64), [B, H, n_c, d]."""
    cp = chunk_pad(chunk_len)
    B, H, _, G = scale.shape
    s = scale.astype(np.float64).reshape(B, H, n_chunks, cp, G)[:, :, :, :chunk_len, :]
    return np.repeat(s.reshape(B, H, n_chunks * chunk_len, G), group, axis=-1)


def step_per_channel_key(scale, chunk_len: int, n_chunks: int, group: int) -> np.ndarray:
    """Per-channel key steps expanded to tokens: Delta_{j,c} (float64), [B, H, n_c, d]."""
    G = -(-chunk_len // group)
    tok_group = np.arange(chunk_len) // group
    B, H, _, d = scale.shape
    s = scale.astype(np.float64).reshape(B, H, n_chunks, G, d)[:, :, :, tok_group, :]
    return s.reshape(B, H, n_chunks * chunk_len, d)
