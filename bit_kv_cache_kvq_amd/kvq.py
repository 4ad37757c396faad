"""ctypes binding of libkvq (include/kvq.h): argument marshalling only.

Every computation runs in the HIP library; this module turns torch tensors into
device pointers and sizes, passes torch's current HIP stream, and raises on a
negative status. Importing it loads ``libkvq.so`` and fails loudly if the library
is missing or was built without an entry point the header declares.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIBRARY overrides the library file (development builds of kernel variants)
library_path = os.environ.get("KVQ_LIBRARY") or os.path.join(_HERE, "libkvq.so")

KVQ_PER_TOKEN, KVQ_PER_CHANNEL, KVQ_PER_TOKEN_GROUP = 0, 1, 2
KVQ_ROLE_KEY, KVQ_ROLE_VALUE = 0, 1
JB_CORR_NONE, JB_CORR_TAYLOR, JB_CORR_EXACT = 0, 1, 2

EXPORTS = ("kvq_chunk_pad", "kvq_window_elems", "kvq_pack", "jb_attn_fwd", "jb_attn_mass",
           "jb_attn_fwd_batch", "jb_attn_mass_batch", "jb_attn_workspace_bytes", "kvq_status_str",
           "jb_attn_fwd_noalloc")
KVQ_BATCH_MAX = 8
JB_NOALLOC_SCRATCH_BYTES = 64 << 20


class KvqError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed with status {status}: {kvq_status_str(status)}")
        self.status = status


class KvqFormat(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("granularity", ctypes.c_int32), ("group", ctypes.c_int32),
                ("hadamard", ctypes.c_int32), ("role", ctypes.c_int32), ("signs", ctypes.c_uint32 * 4)]

    @classmethod
    def make(cls, bits=2, granularity="token", group=128, hadamard=True, role="key", signs=None):
        """signs: None, or d values of +1/-1 (the randomized rotation H diag(s))."""
        gran = {"token": KVQ_PER_TOKEN, "channel": KVQ_PER_CHANNEL, "token_group": KVQ_PER_TOKEN_GROUP}[granularity]
        f = cls(bits, gran, group,
                int(bool(hadamard)), {"key": KVQ_ROLE_KEY, "value": KVQ_ROLE_VALUE}[role])
        for i, w in enumerate(sign_words(signs)):
            f.signs[i] = w
        return f


def sign_words(signs):
    """d values of +1/-1 -> the 4-word mask of kvq_format.signs (bit c set: s_c = -1)."""
    words = [0, 0, 0, 0]
    if signs is None:
        return words
    signs = list(signs)
    if len(signs) > 128 or any(v not in (1, -1) for v in signs):
        raise ValueError("signs must be at most 128 values of +1 or -1")
    for c, v in enumerate(signs):
        if v == -1:
            words[c // 32] |= 1 << (c % 32)
    return words


class JbAttnArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("d", ctypes.c_int32),
                ("n_q", ctypes.c_int32), ("n_r", ctypes.c_int32), ("chunk_len", ctypes.c_int32),
                ("n_chunks", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("k_cur", ctypes.c_void_p), ("v_cur", ctypes.c_void_p),
                ("k_codes", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("k_zero", ctypes.c_void_p),
                ("v_codes", ctypes.c_void_p), ("v_scale", ctypes.c_void_p), ("v_zero", ctypes.c_void_p),
                ("k_fmt", KvqFormat), ("v_fmt", KvqFormat),
                ("softmax_scale", ctypes.c_float), ("correction", ctypes.c_int32),
                ("o", ctypes.c_void_p), ("mass_s", ctypes.c_void_p), ("mass_r", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("window_chunks", ctypes.c_int32)]


def _load():
    if not os.path.exists(library_path):
        raise ImportError(f"libkvq.so not found at {library_path}: run __graft_entry__.build() "
                          "(or python -m bit_kv_cache_kvq_amd.build) first")
    lib = ctypes.CDLL(library_path)
    for name in EXPORTS:
        if not hasattr(lib, name):
            raise ImportError(f"{library_path} does not export {name}")
    lib.kvq_chunk_pad.argtypes = [ctypes.c_int32]
    lib.kvq_chunk_pad.restype = ctypes.c_int32
    lib.kvq_window_elems.argtypes = [ctypes.POINTER(KvqFormat), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t),
                                     ctypes.POINTER(ctypes.c_size_t)]
    lib.kvq_window_elems.restype = ctypes.c_int
    lib.kvq_pack.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                             ctypes.POINTER(KvqFormat), ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.kvq_pack.restype = ctypes.c_int
    for fn in ("jb_attn_fwd", "jb_attn_mass", "jb_attn_fwd_noalloc"):
        getattr(lib, fn).argtypes = [ctypes.POINTER(JbAttnArgs), ctypes.c_void_p]
        getattr(lib, fn).restype = ctypes.c_int
    for fn in ("jb_attn_fwd_batch", "jb_attn_mass_batch"):
        getattr(lib, fn).argtypes = [ctypes.POINTER(JbAttnArgs), ctypes.c_int32, ctypes.c_void_p]
        getattr(lib, fn).restype = ctypes.c_int
    lib.jb_attn_workspace_bytes.argtypes = [ctypes.POINTER(JbAttnArgs)]
    lib.jb_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.kvq_status_str.argtypes = [ctypes.c_int]
    lib.kvq_status_str.restype = ctypes.c_char_p
    return lib


_lib = _load()


def kvq_status_str(status: int) -> str:
    return _lib.kvq_status_str(int(status)).decode()


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, st):
    if st != 0:
        raise KvqError(fn, st)


def kvq_chunk_pad(chunk_len: int) -> int:
    return int(_lib.kvq_chunk_pad(int(chunk_len)))


def window_shapes(fmt: KvqFormat, B: int, H: int, d: int, chunk_len: int, n_chunks: int):
    """(codes shape, scale/zero shape) of a window in the layout kvq.h documents."""
    cw, pe = ctypes.c_size_t(), ctypes.c_size_t()
    _check("kvq_window_elems", _lib.kvq_window_elems(ctypes.byref(fmt), B, H, d, chunk_len, n_chunks,
                                                     ctypes.byref(cw), ctypes.byref(pe)))
    cp = kvq_chunk_pad(chunk_len)
    cpw = 32 // fmt.bits
    if fmt.role == KVQ_ROLE_KEY:
        codes = (B, H, n_chunks * cp, d // cpw)
    else:
        codes = (B, H, n_chunks * cp // 64, d, 64 // cpw)
    if fmt.granularity == KVQ_PER_TOKEN:
        params = (B, H, n_chunks * cp)
    elif fmt.granularity == KVQ_PER_TOKEN_GROUP:
        params = (B, H, n_chunks * cp, d // fmt.group)
    else:
        params = (B, H, n_chunks * (-(-chunk_len // fmt.group)), d)
    assert _prod(codes) == cw.value and _prod(params) == pe.value
    return codes, params


def _prod(s):
    r = 1
    for v in s:
        r *= v
    return r


def alloc_window(fmt: KvqFormat, B, H, d, chunk_len, n_chunks, device="cuda"):
    """Allocate (codes int32, scale int16, zero int16) device tensors for a window."""
    cs, ps = window_shapes(fmt, B, H, d, chunk_len, n_chunks)
    return (torch.empty(cs, dtype=torch.int32, device=device), torch.empty(ps, dtype=torch.int16, device=device),
            torch.empty(ps, dtype=torch.int16, device=device))


def kvq_pack(x, fmt: KvqFormat, n_chunks: int, chunk_idx: int, codes, scale, zero, stream=None):
    """Quantize chunk x (bf16 [B,H,n,d] device tensor) into slot chunk_idx of a window."""
    B, H, n, d = x.shape
    assert x.is_contiguous() and codes.is_contiguous() and scale.is_contiguous() and zero.is_contiguous()
    _check("kvq_pack", _lib.kvq_pack(_ptr(x), B, H, n, d, ctypes.byref(fmt), n_chunks, chunk_idx, _ptr(codes),
                                     _ptr(scale), _ptr(zero), _stream(stream)))


def make_args(q, k_cur, v_cur, k_window, v_window, chunk_len, n_chunks, k_fmt, v_fmt, o=None, mass_s=None,
              mass_r=None, correction=JB_CORR_TAYLOR, softmax_scale=0.0, window_chunks=0):
    """Fill a JbAttnArgs from tensors. k_window / v_window are (codes, scale, zero) or None;
    window_chunks is their per-head chunk capacity when it exceeds n_chunks (0: n_chunks).

    The struct holds raw device pointers; it also keeps references to the tensors, so that
    tensors made inline in the call are not freed (and their memory handed to the next
    allocation, such as the workspace) while the struct is in use.
    The workspace is left empty (the call then runs unsplit); attach_workspace adds it."""
    B, H, n_q, d = q.shape
    n_r = k_cur.shape[2] if k_cur is not None else 0
    kw = k_window if k_window is not None else (None, None, None)
    vw = v_window if v_window is not None else (None, None, None)
    for t in (q, k_cur, v_cur, o, mass_s, mass_r, *kw, *vw):
        assert t is None or t.is_contiguous()
    args = JbAttnArgs(B, H, d, n_q, n_r, chunk_len, n_chunks, _ptr(q), _ptr(k_cur), _ptr(v_cur),
                      _ptr(kw[0]), _ptr(kw[1]), _ptr(kw[2]), _ptr(vw[0]), _ptr(vw[1]), _ptr(vw[2]),
                      k_fmt, v_fmt, float(softmax_scale), int(correction), _ptr(o), _ptr(mass_s), _ptr(mass_r),
                      None, 0, int(window_chunks))
    args.tensors = tuple(t for t in (q, k_cur, v_cur, *kw, *vw, o, mass_s, mass_r) if t is not None)
    return args


def jb_attn_fwd(args: JbAttnArgs, stream=None):
    _check("jb_attn_fwd", _lib.jb_attn_fwd(ctypes.byref(args), _stream(stream)))


def jb_attn_fwd_noalloc(args: JbAttnArgs, stream=None):
    """jb_attn_fwd without allocation: the library's per-device scratch array replaces the
    workspace (args.workspace is ignored)."""
    _check("jb_attn_fwd_noalloc", _lib.jb_attn_fwd_noalloc(ctypes.byref(args), _stream(stream)))


def jb_attn_mass(args: JbAttnArgs, stream=None):
    _check("jb_attn_mass", _lib.jb_attn_mass(ctypes.byref(args), _stream(stream)))


def _batch(fn, calls, stream):
    arr = (JbAttnArgs * len(calls))(*calls)
    _check(fn, getattr(_lib, fn)(arr, len(calls), _stream(stream)))


def jb_attn_fwd_batch(calls, stream=None):
    """Several calls (a sequence of JbAttnArgs) in one launch."""
    _batch("jb_attn_fwd_batch", calls, stream)


def jb_attn_mass_batch(calls, stream=None):
    _batch("jb_attn_mass_batch", calls, stream)


SIZE_MAX = ctypes.c_size_t(-1).value


def jb_attn_workspace_bytes(args: JbAttnArgs) -> int:
    """Workspace bytes the call uses on the current device (0: none); raises on invalid arguments."""
    n = int(_lib.jb_attn_workspace_bytes(ctypes.byref(args)))
    if n == SIZE_MAX:
        raise ValueError("jb_attn_workspace_bytes: invalid attention arguments (jb_attn_fwd would refuse them)")
    return n


def attach_workspace(args: JbAttnArgs, device="cuda"):
    """Allocate the split-window workspace the library asks for on the current device and
    point args at it. Returns the tensor (None when no split is planned); args also keeps a
    reference to it, like to its other tensors."""
    n = jb_attn_workspace_bytes(args)
    if n == 0:
        args.workspace, args.workspace_bytes = None, 0
        args.workspace_tensor = None
        return None
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    args.workspace, args.workspace_bytes = ctypes.c_void_p(ws.data_ptr()), n
    args.workspace_tensor = ws
    return ws


def pack_window(x, chunk_len: int, fmt: KvqFormat, stream=None):
    """Quantize a whole window x (bf16 [B,H,n_chunks*chunk_len,d] device tensor) chunk by chunk.

    Returns freshly allocated (codes, scale, zero). Each chunk is one kvq_pack call.
    """
    B, H, n, d = x.shape
    if n % chunk_len:
        raise ValueError("window is not a whole number of chunks")
    n_chunks = n // chunk_len
    codes, scale, zero = alloc_window(fmt, B, H, d, chunk_len, n_chunks, device=x.device)
    for ci in range(n_chunks):
        chunk = x[:, :, ci * chunk_len:(ci + 1) * chunk_len, :]
        if not chunk.is_contiguous():
            chunk = chunk.contiguous()
        kvq_pack(chunk, fmt, n_chunks, ci, codes, scale, zero, stream)
    return codes, scale, zero
