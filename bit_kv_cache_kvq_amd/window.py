"""A sliding window of quantized chunks for chunk-wise attention.

Chunk-wise autoregressive generation (abstract; §1) denoises one chunk at a time while
attending to earlier chunks through a KV cache. A chunk's keys and values are final once
the chunk is generated: they are quantized once, then read by every denoising step of
the chunks that follow while they stay in the window. ``ChunkWindow`` keeps the last
``capacity`` chunks of one attention layer as a ring of slots in the window layout of
``kvq_pack`` (one allocation per array, never reallocated): the chunk finished t-th goes
to slot t mod capacity, overwriting the oldest one once the ring is full. Calls attend to
the slots in use as chunks 0 .. n_chunks - 1 with ``window_chunks = capacity``; the
attention does not depend on the order of the cached tokens, so no slot is ever moved.

Host bookkeeping only: packing and attention run in libkvq (``kvq_pack``, ``jb_attn_*``);
PyTorch allocates the device memory.
"""
from __future__ import annotations

from . import kvq


def ring_slot(chunks_pushed: int, capacity: int) -> int:
    """Slot of the chunk that is pushed after ``chunks_pushed`` others."""
    if capacity < 1 or chunks_pushed < 0:
        raise ValueError("capacity >= 1 and chunks_pushed >= 0")
    return chunks_pushed % capacity


def window_bytes(fmt: kvq.KvqFormat, B: int, H: int, d: int, chunk_len: int, n_chunks: int) -> int:
    """Device bytes of one quantized window array set (codes + fp16 step + fp16 zero)."""
    cs, ps = kvq.window_shapes(fmt, B, H, d, chunk_len, n_chunks)
    return 4 * kvq._prod(cs) + 2 * 2 * kvq._prod(ps)


class ChunkWindow:
    """The last ``capacity`` chunks of one layer's keys and values, quantized."""

    def __init__(self, B: int, H: int, d: int, chunk_len: int, capacity: int, k_fmt: kvq.KvqFormat,
                 v_fmt: kvq.KvqFormat, device="cuda"):
        if capacity < 1:
            raise ValueError("capacity >= 1")
        self.B, self.H, self.d, self.chunk_len, self.capacity = B, H, d, chunk_len, capacity
        self.k_fmt, self.v_fmt = k_fmt, v_fmt
        self.pushed = 0
        # slots are written by push before any call reads them
        self.k = kvq.alloc_window(k_fmt, B, H, d, chunk_len, capacity, device)
        self.v = kvq.alloc_window(v_fmt, B, H, d, chunk_len, capacity, device)

    @property
    def n_chunks(self) -> int:
        """Chunks in the window (slots 0 .. n_chunks - 1 hold data)."""
        return min(self.pushed, self.capacity)

    def push(self, k_chunk, v_chunk, stream=None) -> int:
        """Quantize a finished chunk (bf16 [B, H, chunk_len, d] device tensors) into the
        next slot; returns the slot."""
        for x in (k_chunk, v_chunk):
            if tuple(x.shape) != (self.B, self.H, self.chunk_len, self.d):
                raise ValueError(f"chunk shape {tuple(x.shape)}")
        slot = ring_slot(self.pushed, self.capacity)
        kvq.kvq_pack(k_chunk, self.k_fmt, self.capacity, slot, *self.k, stream=stream)
        kvq.kvq_pack(v_chunk, self.v_fmt, self.capacity, slot, *self.v, stream=stream)
        self.pushed += 1
        return slot

    def args(self, q, k_cur, v_cur, o=None, mass_s=None, mass_r=None, correction=kvq.JB_CORR_TAYLOR,
             softmax_scale=0.0) -> kvq.JbAttnArgs:
        """Arguments of one attention call of the current chunk over the window."""
        n = self.n_chunks
        return kvq.make_args(q, k_cur, v_cur, self.k if n else None, self.v if n else None, self.chunk_len, n,
                             self.k_fmt, self.v_fmt, o=o, mass_s=mass_s, mass_r=mass_r, correction=correction,
                             softmax_scale=softmax_scale, window_chunks=self.capacity if n else 0)

    def device_bytes(self) -> int:
        """Bytes held by the window's arrays (both tensors, all slots)."""
        return sum(t.numel() * t.element_size() for t in (*self.k, *self.v))
