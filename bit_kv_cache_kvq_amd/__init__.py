"""MI355X-native Jensen-bias-corrected attention over INT2/INT4 quantized KV caches.

The compute path lives in ``libkvq.so`` (HIP kernels for gfx950 behind a C ABI,
declared in ``include/kvq.h``). ``kvq`` is a thin ctypes binding with the same
names; importing it loads the library and raises if it is missing. ``synth``
draws the seeded synthetic workloads. Importing this package itself loads
nothing, so the input generator stays usable on machines without the library.
"""

_BINDING = ("kvq_pack", "jb_attn_fwd", "jb_attn_mass", "jb_attn_workspace_bytes", "kvq_status_str",
            "KvqFormat", "library_path", "window_shapes", "KvqError")


def __getattr__(name):
    if name in _BINDING:
        from . import kvq
        return getattr(kvq, name)
    raise AttributeError(name)
