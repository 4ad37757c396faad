"""kvq_pack on the GPU vs the oracle's quantizer: codes, steps and zero points bit-exact.

The kernel packs whole windows (every head); the oracle re-packs a sample of heads
from the same bf16 bits and every word of those heads must match.
"""
import numpy as np
import pytest

from bit_kv_cache_kvq_amd import synth
from oracle.quant import Format, pack_window
from tests.gpu_util import dev, host_u16, host_u32

pytestmark = pytest.mark.gpu


def _kvq():
    from bit_kv_cache_kvq_amd import kvq
    return kvq


def _check_window(x_bits, chunk_len, bits, gran, group, had, role, heads=None, label="", signs=()):
    kvq = _kvq()
    B, H, n, d = x_bits.shape
    print(f"pack {label}: B={B} H={H} n={n} d={d} chunk={chunk_len} bits={bits} {gran}/{group} had={had} {role}"
          f"{' signs' if signs else ''}", flush=True)
    fmt = kvq.KvqFormat.make(bits, gran, group, had, role, signs or None)
    codes, scale, zero = kvq.pack_window(dev(x_bits), chunk_len, fmt)
    import torch
    torch.cuda.synchronize()
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    ofmt = Format(bits, gran, group, bool(had), role, tuple(signs))
    gw, gs, gz = host_u32(codes), host_u16(scale), host_u16(zero)
    for (b, h) in heads:
        w, s, z = pack_window(x_bits[b:b + 1, h:h + 1], chunk_len, ofmt)
        np.testing.assert_array_equal(gw[b, h], w[0, 0], err_msg=f"codes {label} head {(b, h)}")
        np.testing.assert_array_equal(gs[b, h], s[0, 0].view(np.uint16), err_msg=f"scale {label} head {(b, h)}")
        np.testing.assert_array_equal(gz[b, h], z[0, 0].view(np.uint16), err_msg=f"zero {label} head {(b, h)}")


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_pack_workload_windows(name):
    w = synth.WORKLOADS[name]
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    kc = synth.draw(w, "k_cache")
    _check_window(kc, w.chunk_len, w.bits, w.k_granularity, w.group, 1, "key", heads, f"{name}/K")
    del kc
    vc = synth.draw(w, "v_cache")
    _check_window(vc, w.chunk_len, w.bits, "token", w.group, 1, "value", heads, f"{name}/V")


def test_pack_int4_window():
    w = synth.WORKLOADS["c40"]
    kc = synth.draw(w, "k_cache")
    _check_window(kc, w.chunk_len, 4, "token", 128, 1, "key", [(0, 0), (0, 39)], "c40/K int4")
    vc = synth.draw(w, "v_cache")
    _check_window(vc, w.chunk_len, 4, "token", 128, 1, "value", [(0, 3)], "c40/V int4")


def _edge_input(n_tok, d, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((2, 3, n_tok, d)).astype(np.float32)
    x[..., :3] *= 10
    x[0, 0, 5 % n_tok, :] = 0.75                        # constant token: Delta = 0
    x[0, 1, 7 % n_tok, :] = np.linspace(-3, -2, d)      # range entirely negative: z outside [0, 3]
    x[1, 2, 9 % n_tok, :] = np.linspace(2, 2.001, d)    # tiny positive range
    x[1, 0, :, 7] = 1e-3                        # a near-constant channel (per-channel groups)
    return synth.f32_to_bf16_bits(x)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("chunk_len,n_chunks", [(1, 2), (50, 3), (64, 2), (130, 2), (257, 1)])
@pytest.mark.parametrize("role", ["key", "value"])
@pytest.mark.parametrize("had", [0, 1])
def test_pack_edges_per_token(d, bits, chunk_len, n_chunks, role, had):
    x = _edge_input(chunk_len * n_chunks, d, 100 + chunk_len)
    _check_window(x, chunk_len, bits, "token", 128, had, role, label="edge")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("group", [64, 128])
@pytest.mark.parametrize("chunk_len,n_chunks", [(1, 1), (70, 2), (128, 2), (200, 2), (300, 1)])
@pytest.mark.parametrize("had", [0, 1])
def test_pack_edges_per_channel(d, bits, group, chunk_len, n_chunks, had):
    x = _edge_input(chunk_len * n_chunks, d, 200 + chunk_len)
    _check_window(x, chunk_len, bits, "channel", group, had, "key", label="edge/ch")


def test_pack_rejects_bad_arguments():
    import torch
    kvq = _kvq()
    x = torch.zeros((1, 1, 64, 128), dtype=torch.int16, device="cuda")
    fmt = kvq.KvqFormat.make(2, "token", 128, True, "key")
    codes, scale, zero = kvq.alloc_window(fmt, 1, 1, 128, 64, 1)
    with pytest.raises(kvq.KvqError):
        kvq.kvq_pack(x, fmt, 1, 1, codes, scale, zero)            # chunk_idx out of range
    with pytest.raises(kvq.KvqError):
        kvq.kvq_pack(x, kvq.KvqFormat.make(3, "token", 128, True, "key"), 1, 0, codes, scale, zero)
    with pytest.raises(kvq.KvqError):
        kvq.kvq_pack(x, kvq.KvqFormat.make(2, "channel", 128, True, "value"), 1, 0, codes, scale, zero)
    with pytest.raises(kvq.KvqError):
        kvq.kvq_pack(x[..., :96].contiguous(), fmt, 1, 0, codes, scale, zero)   # d = 96


# randomized rotation H diag(s): codes, steps and zero points bit-exact with the oracle
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits,gran,role", [(2, "token", "key"), (4, "token", "value"), (2, "channel", "key")])
def test_pack_randomized_rotation(d, bits, gran, role):
    w = synth.Workload("signs", B=1, H=2, d=d, n_q=64, chunk_len=200, n_chunks=2, seed=8,
                       k_dist="t3" if gran == "channel" else "outlier")
    x = synth.draw(w, "k_cache")
    s = synth.draw_signs(d, 5, "k")
    _check_window(x, w.chunk_len, bits, gran, 128, 1, role, None, f"signs d{d}", signs=s)


@pytest.mark.parametrize("g", [32, 64])
@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("role", ["key", "value"])
def test_pack_token_group(g, bits, role):
    # group-wise per token (channel groups of g, one step and zero point each), on a ragged
    # chunk length, with the degenerate-range and outlier rows of the edge input
    x = _edge_input(3 * 97, 128, 31 + g + bits)
    _check_window(x, 97, bits, "token_group", g, 1, role, label=f"token_group g={g}")
    _check_window(x[..., :64], 97, bits, "token_group", 32, 0, role, label=f"token_group d=64 g=32")
    w = synth.WORKLOADS["c24"]
    xc = synth.draw(w, "k_cache" if role == "key" else "v_cache", heads=[(0, 0), (0, 23)])[None]
    _check_window(xc, w.chunk_len, bits, "token_group", g, 1, role, label=f"c24 heads token_group g={g}")
