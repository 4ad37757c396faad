"""Build libkvq.so (HIP, gfx950) in-tree with hipcc.

The quantizer's translation unit is compiled with -ffp-contract=off and correctly
rounded float32 division, because its codes and fp16 steps must follow one exact
float32 operation order. All HIP code is compiled without packed-fp32 instructions.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkvq.so")

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fhip-fp32-correctly-rounded-divide-sqrt", "-Wall", "-Wno-unused-function"]
UNITS = {
    "pack.hip": ["-ffp-contract=off"],
    "attn.hip": [],
}


def hipcc() -> str:
    return os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    """Compile every HIP unit and link libkvq.so next to this file; returns its path."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="kvq_build_") as tmp:
        objs = []
        for unit, extra in UNITS.items():
            obj = os.path.join(tmp, unit + ".o")
            cmd = [cc, *COMMON, *extra, "-c", os.path.join(CSRC, unit), "-o", obj]
            _run(cmd, verbose)
            objs.append(obj)
        out = os.path.join(tmp, "libkvq.so")
        _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", out], verbose)
        staged = LIB + ".tmp"
        shutil.copyfile(out, staged)
        os.replace(staged, LIB)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(ln for ln in (r.stderr or "").splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose=True))
