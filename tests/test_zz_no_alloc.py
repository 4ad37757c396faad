"""jb_attn_fwd_noalloc (the forward pass for callers that cannot allocate) against
jb_attn_fwd with a workspace the caller allocated: identical outputs, on two calls in a row
on one device, the second smaller than the first (the scratch array keeps the first call's
contents), plus the oracle on both; and the refusal of a call whose plan needs more scratch
than the array holds."""
import ctypes

import numpy as np
import pytest
import torch

from bit_kv_cache_kvq_amd import synth
from tests.gpu_util import assert_attention_close, assert_mass_close, dev, lib_formats, oracle_formats

import oracle

pytestmark = pytest.mark.gpu


def _setup(w):
    from bit_kv_cache_kvq_amd import kvq
    x = synth.draw_all(w)
    kf, vf = lib_formats(w)
    t = {"q": dev(x["q"]), "kr": dev(x["k_cur"]), "vr": dev(x["v_cur"])}
    t["kwin"] = kvq.pack_window(dev(x["k_cache"]), w.chunk_len, kf)
    t["vwin"] = kvq.pack_window(dev(x["v_cache"]), w.chunk_len, vf)

    def outputs():
        o = torch.full((w.B, w.H, w.n_q, w.d), float("nan"), dtype=torch.float32, device="cuda")
        ms = torch.full((w.B, w.H, w.n_q), float("nan"), dtype=torch.float32, device="cuda")
        mr = torch.full((w.B, w.H, w.n_q), float("nan"), dtype=torch.float32, device="cuda")
        a = kvq.make_args(t["q"], t["kr"], t["vr"], t["kwin"], t["vwin"], w.chunk_len, w.n_chunks, kf, vf,
                          o=o, mass_s=ms, mass_r=mr, correction=kvq.JB_CORR_TAYLOR)
        return a, (o, ms, mr)

    return x, t, outputs


def _run_pair(w):
    """Returns (need, with-workspace outputs, no-allocation outputs) as numpy arrays."""
    from bit_kv_cache_kvq_amd import kvq
    x, t, outputs = _setup(w)
    a1, out1 = outputs()
    need = kvq.jb_attn_workspace_bytes(a1)
    ws = kvq.attach_workspace(a1)
    kvq.jb_attn_fwd(a1)
    a2, out2 = outputs()
    a2.workspace, a2.workspace_bytes = None, 0
    st = kvq._lib.jb_attn_fwd_noalloc(ctypes.byref(a2), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, kvq.kvq_status_str(st)
    torch.cuda.synchronize()
    del ws
    return x, need, [v.cpu().numpy() for v in out1], [v.cpu().numpy() for v in out2]


# a split call (few query blocks for the device: partial records in the scratch array), then
# a smaller few-query call (the decode path's records, written over the first call's)
CASES = [
    synth.Workload("noalloc_split", B=1, H=4, d=128, n_q=300, chunk_len=256, n_chunks=3, seed=81),
    synth.Workload("noalloc_decode", B=1, H=2, d=128, n_q=16, chunk_len=200, n_chunks=2, seed=82),
]


def test_noalloc_matches_workspace_call_twice():
    from bit_kv_cache_kvq_amd import kvq
    needs = []
    for w in CASES:
        print(f"noalloc {w.name}: B={w.B} H={w.H} n_q={w.n_q} window {w.n_chunks}x{w.chunk_len}", flush=True)
        x, need, ref, got = _run_pair(w)
        assert 0 < need <= kvq.JB_NOALLOC_SCRATCH_BYTES, need
        needs.append(need)
        for r, g in zip(ref, got):
            np.testing.assert_array_equal(g, r)
        kf, vf = oracle_formats(w)
        Or, PSr, PRr, _ = oracle.reference_call(x["q"], x["k_cache"], x["v_cache"], x["k_cur"], x["v_cur"],
                                                chunk_len=w.chunk_len, k_fmt=kf, v_fmt=vf, correction="taylor")
        assert_attention_close(got[0], Or, f"noalloc {w.name}")
        assert_mass_close(got[1], got[2], PSr, PRr, f"noalloc {w.name}")
    assert needs[1] < needs[0]


def test_noalloc_refuses_calls_beyond_the_scratch():
    from bit_kv_cache_kvq_amd import kvq
    # 256-query blocks of many heads with a short window: the device takes the grid in one
    # round, so the call splits, and its partial records outgrow the array
    for H in range(150, 260, 5):
        w = synth.Workload("noalloc_big", B=1, H=H, d=128, n_q=256, chunk_len=64, n_chunks=3, seed=83)
        kf, vf = lib_formats(w)
        z = lambda *s, dt=torch.int16: torch.zeros(s, dtype=dt, device="cuda")
        kc, ks, kz = kvq.alloc_window(kf, w.B, w.H, w.d, w.chunk_len, w.n_chunks)
        vc, vs, vz = kvq.alloc_window(vf, w.B, w.H, w.d, w.chunk_len, w.n_chunks)
        q, kr, vr = z(1, H, 256, 128), z(1, H, 256, 128), z(1, H, 256, 128)
        o = z(1, H, 256, 128, dt=torch.float32)
        a = kvq.make_args(q, kr, vr, (kc, ks, kz), (vc, vs, vz), w.chunk_len, w.n_chunks, kf, vf, o=o)
        need = kvq.jb_attn_workspace_bytes(a)
        if need > kvq.JB_NOALLOC_SCRATCH_BYTES:
            print(f"noalloc refusal: H={H} needs {need} bytes", flush=True)
            o.fill_(7.0)
            st = kvq._lib.jb_attn_fwd_noalloc(ctypes.byref(a), None)
            torch.cuda.synchronize()
            assert st == -5, st
            assert torch.all(o == 7.0)  # nothing launched
            return
    pytest.skip("no shape in the range needs more than the scratch array on this device")
