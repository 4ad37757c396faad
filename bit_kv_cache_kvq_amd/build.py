"""Build libkvq.so (HIP, gfx950) in-tree with hipcc.

The quantizer's translation unit is compiled with -ffp-contract=off and correctly
rounded float32 division, because its codes and fp16 steps must follow one exact
float32 operation order. All HIP code is compiled without packed-fp32 instructions.
The host-only unit (argument validation and launch planning) is plain C++ built with
the host compiler; the translation units compile in parallel.

The attention unit is also compiled to device assembly, which the build checks: the
gfx950 MX conversions (``v_cvt_scalef32_*``) write part of their result before they have
read all of their sources, and the compiler does not keep the two apart, so the kernels
are written to keep every such source live past its conversion; a build whose code has
a conversion writing over one of its own sources is refused.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

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
HOST_UNITS = ["host.cpp"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    return os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    """Compile every HIP unit and link libkvq.so next to this file; returns its path."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="kvq_build_") as tmp:
        jobs = []
        for unit, extra in UNITS.items():
            obj = os.path.join(tmp, unit + ".o")
            jobs.append(([cc, *COMMON, *extra, "-c", os.path.join(CSRC, unit), "-o", obj], obj))
        for unit in HOST_UNITS:
            obj = os.path.join(tmp, unit + ".o")
            jobs.append((["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, unit), "-o", obj], obj))
        asm = os.path.join(tmp, "attn.s")
        asm_job = ([cc, *COMMON, "--cuda-device-only", "-S", os.path.join(CSRC, "attn.hip"), "-o", asm], None)
        with ThreadPoolExecutor(max_workers=len(jobs) + 1) as ex:
            list(ex.map(lambda j: _run(j[0], verbose), jobs + [asm_job]))
        bad = overlapping_conversions(open(asm).read())
        if bad:
            raise RuntimeError("build refused: MX conversions writing over their own sources:\n" + "\n".join(bad))
        objs = [o for _, o in jobs]
        out = os.path.join(tmp, "libkvq.so")
        _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", out], verbose)
        staged = LIB + ".tmp"
        shutil.copyfile(out, staged)
        os.replace(staged, LIB)
    return LIB


def _vgprs(operand: str) -> set:
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", operand.strip())
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", operand.strip())
    return {int(m.group(1))} if m else set()


def overlapping_conversions(asm: str) -> list:
    """Lines of gfx950 assembly whose v_cvt_scalef32_* result registers overlap a source."""
    bad = []
    for line in asm.splitlines():
        m = re.match(r"\s+(v_cvt_scalef32_\S+)\s+(.*)", line)
        if not m:
            continue
        ops = re.split(r",\s*", m.group(2).split(";")[0])
        dst, srcs = _vgprs(ops[0]), set().union(*[_vgprs(o) for o in ops[1:]])
        if dst & srcs:
            bad.append(line.strip())
    return bad


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
