"""Helpers shared by the GPU parity tests: device upload and the tolerance checks."""
import numpy as np
import torch

from oracle.quant import Format

# Attention output tolerance (relative to the RMS of the oracle's output over the checked rows)
MAX_ERR = 1e-2
MEAN_ERR = 1e-3
MASS_ERR = 1e-3


def dev(a):
    """bf16/fp16 bit arrays (uint16) -> int16 device tensor with the same bits."""
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_u16(t):
    return t.cpu().numpy().view(np.uint16)


def host_u32(t):
    return t.cpu().numpy().view(np.uint32)


def oracle_formats(w, k_had=True, v_had=True, bits=None, k_signs=(), v_signs=()):
    b = bits or w.bits
    kf = Format(b, w.k_granularity, w.group, k_had, "key", tuple(k_signs))
    vf = Format(b, w.v_granularity, w.group, v_had, "value", tuple(v_signs))
    return kf, vf


def lib_formats(w, k_had=True, v_had=True, bits=None, k_signs=(), v_signs=()):
    from bit_kv_cache_kvq_amd import kvq
    b = bits or w.bits
    kf = kvq.KvqFormat.make(b, w.k_granularity, w.group, k_had, "key", k_signs or None)
    vf = kvq.KvqFormat.make(b, w.v_granularity, w.group, v_had, "value", v_signs or None)
    return kf, vf


def assert_attention_close(o_gpu, o_ref, label=""):
    err = np.abs(o_gpu.astype(np.float64) - o_ref)
    rms = np.sqrt(np.mean(o_ref ** 2))
    mx, mean = err.max() / rms, err.mean() / rms
    print(f"[{label}] max|err|/rms={mx:.3e} mean|err|/rms={mean:.3e}", flush=True)
    assert np.all(np.isfinite(o_gpu))
    assert mx <= MAX_ERR, (label, mx)
    assert mean <= MEAN_ERR, (label, mean)
    return mx, mean


def assert_mass_close(ps, pr, ps_ref, pr_ref, label=""):
    e = max(np.abs(ps - ps_ref).max(), np.abs(pr - pr_ref).max())
    print(f"[{label}] mass max err={e:.3e}", flush=True)
    assert e <= MASS_ERR, (label, e)
    assert np.abs(ps.astype(np.float64) + pr - 1).max() <= 1e-6
