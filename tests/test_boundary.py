"""The C ABI: libkvq.so loads, exports every function include/kvq.h declares, and its
host-side validation rejects bad arguments before anything is launched (no GPU needed)."""
import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "kvq.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def kvq():
    from bit_kv_cache_kvq_amd import kvq as mod
    return mod


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for fn in ["kvq_pack", "jb_attn_fwd", "jb_attn_mass", "jb_attn_workspace_bytes", "kvq_status_str",
               "kvq_chunk_pad", "kvq_window_elems", "jb_attn_fwd_batch", "jb_attn_mass_batch"]:
        assert fn in names


def test_library_exports_every_declared_symbol(kvq):
    lib = ctypes.CDLL(kvq.library_path)
    for fn in _declared_functions():
        assert hasattr(lib, fn), fn
    assert set(_declared_functions()) <= set(kvq.EXPORTS)


def test_struct_layouts_match_header(kvq):
    # five int32 fields and four uint32 sign words; no hidden padding on x86-64
    assert ctypes.sizeof(kvq.KvqFormat) == 36
    assert kvq.KvqFormat.signs.offset == 20
    off = kvq.JbAttnArgs.q.offset
    assert off == 32  # 7 int32 = 28 bytes, pointer aligned to 8
    assert kvq.JbAttnArgs.window_chunks.offset == kvq.JbAttnArgs.workspace_bytes.offset + 8


def test_geometry(kvq):
    assert kvq.kvq_chunk_pad(1) == 64 and kvq.kvq_chunk_pad(64) == 64 and kvq.kvq_chunk_pad(4680) == 4736
    assert kvq.kvq_chunk_pad(0) == 0
    f = kvq.KvqFormat.make(2, "token", 128, True, "key")
    assert kvq.window_shapes(f, 1, 40, 128, 4680, 8) == ((1, 40, 37888, 8), (1, 40, 37888))
    f = kvq.KvqFormat.make(2, "token", 128, True, "value")
    assert kvq.window_shapes(f, 1, 40, 128, 4680, 8) == ((1, 40, 592, 128, 4), (1, 40, 37888))
    f = kvq.KvqFormat.make(4, "channel", 128, True, "key")
    assert kvq.window_shapes(f, 1, 40, 128, 4680, 8) == ((1, 40, 37888, 16), (1, 40, 296, 128))
    f = kvq.KvqFormat.make(2, "token_group", 32, True, "value")
    assert kvq.window_shapes(f, 1, 40, 128, 4680, 8) == ((1, 40, 592, 128, 4), (1, 40, 37888, 4))
    # a channel group must be narrower than d (a group of d channels is the per-token format)
    cw, pe = ctypes.c_size_t(), ctypes.c_size_t()
    f64 = kvq.KvqFormat.make(2, "token_group", 64, True, "key")
    assert kvq._lib.kvq_window_elems(ctypes.byref(f64), 1, 1, 64, 128, 1, ctypes.byref(cw), ctypes.byref(pe)) == -3
    assert kvq._lib.kvq_window_elems(ctypes.byref(f64), 1, 1, 128, 128, 1, ctypes.byref(cw), ctypes.byref(pe)) == 0
    f = kvq.KvqFormat.make(4, "token_group", 64, True, "key")
    assert kvq.window_shapes(f, 2, 3, 128, 100, 2) == ((2, 3, 256, 16), (2, 3, 256, 2))
    # bytes per token and head at d=128: INT2 32 + 4, INT4 64 + 4 (codes + fp16 step and zero)
    assert 128 * 2 // 8 + 4 == 36 and 128 * 4 // 8 + 4 == 68


def test_status_strings(kvq):
    for st in range(0, -7, -1):
        assert kvq.kvq_status_str(st) != "unknown status"
    assert kvq.kvq_status_str(-99) == "unknown status"


def test_pack_validation_without_launch(kvq):
    lib = kvq._lib
    p = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    f = kvq.KvqFormat.make(2, "token", 128, True, "key")
    call = lambda fmt, *a: lib.kvq_pack(*a[:5], ctypes.byref(fmt) if fmt else None, *a[5:])
    assert call(f, None, 1, 1, 64, 128, 1, 0, p, p, p, None) == -1           # null input
    assert call(None, p, 1, 1, 64, 128, 1, 0, p, p, p, None) == -1           # null format
    assert call(f, p, 1, 1, 64, 96, 1, 0, p, p, p, None) == -2               # d
    assert call(f, p, 0, 1, 64, 128, 1, 0, p, p, p, None) == -2              # B
    assert call(f, p, 1, 1, 64, 128, 2, 2, p, p, p, None) == -2              # chunk_idx
    assert call(kvq.KvqFormat.make(3, "token", 128, True, "key"), p, 1, 1, 64, 128, 1, 0, p, p, p, None) == -3
    assert call(kvq.KvqFormat.make(2, "channel", 96, True, "key"), p, 1, 1, 64, 128, 1, 0, p, p, p, None) == -3
    assert call(kvq.KvqFormat.make(2, "channel", 128, True, "value"), p, 1, 1, 64, 128, 1, 0, p, p, p, None) == -3
    assert call(kvq.KvqFormat.make(2, "token_group", 16, True, "key"), p, 1, 1, 64, 128, 1, 0, p, p, p, None) == -3
    assert call(kvq.KvqFormat.make(2, "token_group", 64, True, "key"), p, 1, 1, 64, 64, 1, 0, p, p, p, None) == -3
    q = ctypes.c_void_p(18)
    assert call(f, q, 1, 1, 64, 128, 1, 0, p, p, p, None) == -4              # misaligned
    nosign = kvq.KvqFormat.make(2, "token", 128, False, "key", [-1] + [1] * 127)
    assert call(nosign, p, 1, 1, 64, 128, 1, 0, p, p, p, None) == -3         # signs without rotation
    wide = kvq.KvqFormat.make(2, "token", 128, True, "key", [1] * 127 + [-1])
    assert call(wide, p, 1, 1, 64, 64, 1, 0, p, p, p, None) == -3            # sign past channel d


def test_attn_validation_without_launch(kvq):
    lib = kvq._lib
    kf = kvq.KvqFormat.make(2, "token", 128, True, "key")
    vf = kvq.KvqFormat.make(2, "token", 128, True, "value")
    P = 4096

    def args(**kw):
        a = kvq.JbAttnArgs(1, 1, 128, 64, 64, 64, 1, P, P, P, P, P, P, P, P, P, kf, vf, 0.0, 1, P, None, None,
                           None, 0)
        for k, v in kw.items():
            setattr(a, k, v)
        return a

    fwd = lambda a: lib.jb_attn_fwd(ctypes.byref(a), None)
    mass = lambda a: lib.jb_attn_mass(ctypes.byref(a), None)
    assert lib.jb_attn_fwd(None, None) == -1
    assert fwd(args(d=96)) == -2
    assert fwd(args(n_q=0)) == -2
    assert fwd(args(n_chunks=0, n_r=0)) == -2
    assert fwd(args(correction=7)) == -3
    assert fwd(args(correction=3)) == -3
    assert fwd(args(window_chunks=-1)) == -2
    assert fwd(args(n_chunks=2, window_chunks=1)) == -2     # fewer slots than chunks attended
    assert fwd(args(n_chunks=2, window_chunks=3, o=None)) == -1
    assert fwd(args(correction=2, o=None)) == -1   # JB_CORR_EXACT passes the option check
    assert fwd(args(k_fmt=kvq.KvqFormat.make(2, "token", 128, False, "key", [-1] * 128))) == -3
    assert fwd(args(d=64, v_fmt=kvq.KvqFormat.make(2, "token", 128, True, "value", [1] * 127 + [-1]))) == -3
    assert fwd(args(k_fmt=kvq.KvqFormat.make(2, "token", 128, True, "key", [-1] * 128), o=None)) == -1
    assert fwd(args(v_fmt=kvq.KvqFormat.make(4, "token", 128, True, "value"))) == -3
    assert fwd(args(v_fmt=kf)) == -3
    tg = lambda g, role, d=128: kvq.KvqFormat.make(2, "token_group", g, True, role)
    assert fwd(args(k_fmt=tg(32, "key"))) == -3                                  # values must be group-wise too
    assert fwd(args(k_fmt=tg(32, "key"), v_fmt=tg(64, "value"))) == -3          # one group size
    assert fwd(args(k_fmt=tg(32, "key"), v_fmt=tg(32, "value"), correction=2, o=None)) == -1  # exact: the format passes
    assert fwd(args(d=64, k_fmt=tg(64, "key"), v_fmt=tg(64, "value"))) == -3   # a group narrower than d
    assert fwd(args(k_fmt=tg(32, "key"), v_fmt=tg(32, "value"), o=None)) == -1  # the format passes
    assert fwd(args(o=None)) == -1
    assert fwd(args(k_codes=None)) == -1
    assert fwd(args(mass_s=P)) == -1            # masses come in pairs
    assert fwd(args(q=P + 2)) == -4
    assert fwd(args(softmax_scale=-1.0)) == -2
    assert mass(args()) == -1                   # mass needs mass_s / mass_r
    assert lib.jb_attn_workspace_bytes(ctypes.byref(args())) == 0   # no device here: no split planned
    size_max = ctypes.c_size_t(-1).value
    assert lib.jb_attn_workspace_bytes(ctypes.byref(args(softmax_scale=-1.0))) == size_max  # invalid arguments
    assert lib.jb_attn_workspace_bytes(None) == size_max
    with pytest.raises(ValueError):
        kvq.jb_attn_workspace_bytes(args(q=P + 2, o=None, mass_s=None))
    assert kvq.kvq_status_str(-5).startswith("workspace smaller")


def test_batch_validation_without_launch(kvq):
    lib = kvq._lib
    kf = kvq.KvqFormat.make(2, "token", 128, True, "key")
    vf = kvq.KvqFormat.make(2, "token", 128, True, "value")
    P = 4096

    def args(**kw):
        a = kvq.JbAttnArgs(1, 1, 128, 64, 64, 64, 1, P, P, P, P, P, P, P, P, P, kf, vf, 0.0, 1, P, None, None,
                           None, 0)
        for k, v in kw.items():
            setattr(a, k, v)
        return a

    def batch(calls, n=None):
        arr = (kvq.JbAttnArgs * len(calls))(*calls)
        return lib.jb_attn_fwd_batch(arr, len(calls) if n is None else n, None)

    assert lib.jb_attn_fwd_batch(None, 1, None) == -1
    assert batch([args()], n=0) == -2
    assert batch([args()] * 9) == -2                                   # more than KVQ_BATCH_MAX
    assert batch([args(), args(o=None)]) == -1                        # a call's own validation
    tgk, tgv = kvq.KvqFormat.make(2, "token_group", 32, True, "key"), kvq.KvqFormat.make(2, "token_group", 32, True, "value")
    assert batch([args(k_fmt=tgk, v_fmt=tgv), args()]) == -3            # group-wise and per-token mixed
    tgk64, tgv64 = kvq.KvqFormat.make(2, "token_group", 64, True, "key"), kvq.KvqFormat.make(2, "token_group", 64, True, "value")
    assert batch([args(k_fmt=tgk, v_fmt=tgv), args(k_fmt=tgk64, v_fmt=tgv64)]) == -3  # two group sizes
    assert batch([args(), args(d=64, k_fmt=kvq.KvqFormat.make(2, "token", 128, True, "key"))]) == -3
    assert batch([args(), args(correction=2)]) == -3                  # exact and Taylor mixed
    assert batch([args(), args(k_fmt=kvq.KvqFormat.make(4, "token", 128, True, "key"),
                               v_fmt=kvq.KvqFormat.make(4, "token", 128, True, "value"))]) == -3
    assert kvq.KVQ_BATCH_MAX == 8


def test_sign_words(kvq):
    assert kvq.sign_words(None) == [0, 0, 0, 0]
    assert kvq.sign_words([1, -1, 1, -1] + [1] * 60) == [0b1010, 0, 0, 0]
    assert kvq.sign_words([1] * 100 + [-1] + [1] * 27) == [0, 0, 0, 1 << 4]
    with pytest.raises(ValueError):
        kvq.sign_words([0] * 64)


def test_window_ring_bookkeeping(kvq):
    from bit_kv_cache_kvq_amd import window
    assert [window.ring_slot(t, 3) for t in range(7)] == [0, 1, 2, 0, 1, 2, 0]
    with pytest.raises(ValueError):
        window.ring_slot(0, 0)
    # c40 window (8 chunks of 4680 tokens, 40 heads, d 128): INT2 K+V against INT4 and bf16
    fk = lambda b: kvq.KvqFormat.make(b, "token", 128, True, "key")
    fv = lambda b: kvq.KvqFormat.make(b, "token", 128, True, "value")
    w2 = window.window_bytes(fk(2), 1, 40, 128, 4680, 8) + window.window_bytes(fv(2), 1, 40, 128, 4680, 8)
    w4 = window.window_bytes(fk(4), 1, 40, 128, 4680, 8) + window.window_bytes(fv(4), 1, 40, 128, 4680, 8)
    bf16 = 2 * 40 * 8 * 4680 * 128 * 2
    assert w2 == 2 * 40 * 8 * 4736 * (32 + 4)      # padded tokens: 32 code bytes + fp16 step and zero
    assert abs(w2 / w4 - 0.529) < 1e-3 and w2 / bf16 < 0.15


def test_build_refuses_conversions_over_their_sources():
    # the build's check of the device assembly (MX conversions whose result overlaps a
    # source register read the overwritten values; the build refuses such code)
    from bit_kv_cache_kvq_amd.build import overlapping_conversions
    asm = "\n".join([
        "\tv_cvt_scalef32_2xpk16_fp6_f32 v[32:37], v[2:17], v[18:33], s0",   # overlaps v32, v33
        "\tv_cvt_scalef32_2xpk16_fp6_f32 v[34:39], v[2:17], v[18:33], v41",
        "\tv_cvt_scalef32_pk32_f32_fp6 v[0:31], v[32:37], s0 ; comment v[0:40]",
        "\tv_cvt_scalef32_pk32_f32_fp6 v[0:31], v[30:35], v36",              # overlaps v30, v31
        "\tv_mov_b32 v1, v1",
    ])
    assert overlapping_conversions(asm) == ["v_cvt_scalef32_2xpk16_fp6_f32 v[32:37], v[2:17], v[18:33], s0",
                                            "v_cvt_scalef32_pk32_f32_fp6 v[0:31], v[30:35], v36"]


def test_args_keep_their_tensors_alive(kvq):
    # the struct holds raw pointers: tensors made inline in make_args must live as long as
    # the struct (else their memory goes to the next allocation, e.g. the workspace)
    import gc
    import weakref

    import torch
    fmt = kvq.KvqFormat.make(2, "token", 128, True, "key")
    vfmt = kvq.KvqFormat.make(2, "token", 128, True, "value")
    refs = []

    def t(*shape, dtype=torch.int16):
        x = torch.zeros(*shape, dtype=dtype)
        refs.append(weakref.ref(x))
        return x

    a = kvq.make_args(t(1, 1, 64, 128), t(1, 1, 64, 128), t(1, 1, 64, 128), (t(1, 1, 64, 8, dtype=torch.int32),
                      t(1, 1, 64), t(1, 1, 64)), (t(1, 1, 64, 8, dtype=torch.int32), t(1, 1, 64), t(1, 1, 64)),
                      64, 1, fmt, vfmt, o=t(1, 1, 64, 128, dtype=torch.float32))
    gc.collect()
    assert all(r() is not None for r in refs)
    assert a.q == a.tensors[0].data_ptr()
    del a
    gc.collect()
    assert all(r() is None for r in refs)
