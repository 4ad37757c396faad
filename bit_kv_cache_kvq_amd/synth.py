"""Seeded synthetic workloads for chunk-wise attention over a quantized KV cache.

This module draws inputs only. It holds none of the method's arithmetic (no
rotation, quantization, correction or attention) and imports nothing from the
HIP binding or from the oracle, so both sides can be fed from it.

The paper (*Quantized Keys Steal Attention: Bias Correction for KV-Cache
Compression in Video Diffusion*, Tuncer, Becker, Pfeil, arXiv 2605.26266)
evaluates on chunk-wise autoregressive video models (abstract; §1) whose
weights and prompts are not available here. The workloads below stand in for
them with video-shaped sizes: a latent frame of 30x52 = 1,560 patches, chunks of
one or three frames, and a sliding window of previous chunks (§1, the
sliding-window discussion next to Fig. 3). Keys carry channel-wise outliers,
the property that motivates the Hadamard rotation (§3 "Hadamard rotation").

Recipe (fixed, so that every run and both sides see identical bits):

* every tensor is drawn per (tensor, b, h) slice from its own PCG64 stream
  ``np.random.default_rng([seed, tensor_id, b, h])`` so slices can be drawn in
  parallel threads without changing any value;
* N(0,1) draws are float32 ``standard_normal``; Student-t(3) draws are float64
  ``standard_t(3)`` cast to float32;
* outlier key channels 0..n_outlier-1 are multiplied by ``outlier_scale`` in
  float32, for cached and current keys alike;
* float32 -> bfloat16 is round-to-nearest-even on the bit pattern.

Arrays are returned as ``uint16`` bfloat16 bit patterns, shape ``[B, H, n, d]``.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

TENSOR_IDS = {"q": 0, "k_cache": 1, "v_cache": 2, "k_cur": 3, "v_cur": 4}


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and input distribution of one chunk-attention call."""

    name: str
    B: int
    H: int
    d: int
    n_q: int            # current-chunk queries (== current-chunk keys)
    chunk_len: int      # tokens per cached chunk
    n_chunks: int       # cached chunks in the sliding window
    k_dist: str = "outlier"   # "outlier": N(0,1) with scaled channels; "t3": Student-t(3)
    n_outlier: int = 4
    outlier_scale: float = 10.0
    k_granularity: str = "token"  # "token" | "channel" | "token_group"
    group: int = 128              # tokens per per-channel key group, or channels per token group
    bits: int = 2
    masses: bool = False
    seed: int = 0

    @property
    def v_granularity(self) -> str:
        """Values are per token, or group-wise per token together with group-wise keys."""
        return "token_group" if self.k_granularity == "token_group" else "token"

    @property
    def n_r(self) -> int:
        return self.n_q

    @property
    def n_c(self) -> int:
        return self.chunk_len * self.n_chunks

    @property
    def bh(self) -> int:
        return self.B * self.H

    def flops(self) -> float:
        """Algorithmic FLOP of one attention call: QK^T and PV over cached + current keys."""
        return 4.0 * self.n_q * (self.n_c + self.n_r) * self.d * self.bh

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny one the oracle finishes in well under a second,
# one-frame chunks with a 4-chunk window, three-frame chunks with an 8-chunk
# window (per-token and per-channel keys), and a long window of 16 frames of
# 68x120 patches.
WORKLOADS = {
    "tiny": Workload("tiny", B=1, H=2, d=64, n_q=128, chunk_len=128, n_chunks=2,
                     n_outlier=2, outlier_scale=8.0),
    "c24": Workload("c24", B=1, H=24, d=128, n_q=1560, chunk_len=1560, n_chunks=4),
    "c40": Workload("c40", B=1, H=40, d=128, n_q=4680, chunk_len=4680, n_chunks=8),
    "c40_perch": Workload("c40_perch", B=1, H=40, d=128, n_q=4680, chunk_len=4680, n_chunks=8,
                          k_dist="t3", k_granularity="channel", group=128),
    # the per-channel workload with the window packed as one sequence: key groups of 128
    # tokens run over the whole window, across the boundaries of its 8 chunks (same data)
    "c40_perch_span": Workload("c40_perch_span", B=1, H=40, d=128, n_q=4680, chunk_len=37440, n_chunks=1,
                               k_dist="t3", k_granularity="channel", group=128),
    # the c40 shape with group-wise per-token keys and values (32 channels per group)
    "c40_tgroup": Workload("c40_tgroup", B=1, H=40, d=128, n_q=4680, chunk_len=4680, n_chunks=8,
                           k_granularity="token_group", group=32),
    "long": Workload("long", B=2, H=48, d=128, n_q=8160, chunk_len=8160, n_chunks=16, masses=True),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw_slice(w: Workload, tensor: str, b: int, h: int, n: int) -> np.ndarray:
    rng = np.random.default_rng([w.seed, TENSOR_IDS[tensor], b, h])
    is_key = tensor in ("k_cache", "k_cur")
    if is_key and w.k_dist == "t3":
        x = rng.standard_t(3, size=(n, w.d)).astype(np.float32)
    else:
        x = rng.standard_normal((n, w.d), dtype=np.float32)
        if is_key and w.k_dist == "outlier" and w.n_outlier > 0:
            x[:, : w.n_outlier] *= np.float32(w.outlier_scale)
    return f32_to_bf16_bits(x)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def draw(w: Workload, tensor: str, heads: list[tuple[int, int]] | None = None) -> np.ndarray:
    """Draw one tensor of workload ``w`` as bf16 bits.

    ``heads`` restricts the draw to the listed (b, h) pairs (result shape
    ``[len(heads), n, d]``); the values equal the corresponding slices of the
    full tensor.
    """
    n = {"q": w.n_q, "k_cache": w.n_c, "v_cache": w.n_c, "k_cur": w.n_r, "v_cur": w.n_r}[tensor]
    full = heads is None
    if full:
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    out = np.empty((len(heads), n, w.d), dtype=np.uint16)

    def job(i):
        b, h = heads[i]
        out[i] = _draw_slice(w, tensor, b, h, n)

    if len(heads) == 1:
        job(0)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(job, range(len(heads))))
    if full:
        return out.reshape(w.B, w.H, n, w.d)
    return out


def draw_all(w: Workload, heads: list[tuple[int, int]] | None = None) -> dict[str, np.ndarray]:
    """All five inputs of a call: q, k_cache, v_cache, k_cur, v_cur (bf16 bits)."""
    return {t: draw(w, t, heads) for t in TENSOR_IDS}


def draw_signs(d: int, seed: int, tensor: str = "k") -> tuple:
    """A sign vector for a randomized Hadamard rotation H diag(s) (§3 names the
    randomized rotation): d values of +1/-1, each -1 with probability 1/2, from
    ``np.random.default_rng([seed, 100 + id])`` with id 0 for keys and 1 for values."""
    rng = np.random.default_rng([seed, 100 + {"k": 0, "v": 1}[tensor]])
    return tuple(int(v) for v in np.where(rng.integers(0, 2, d) == 1, -1, 1))
