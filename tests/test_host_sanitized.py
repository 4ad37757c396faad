"""Host-side validation and launch planning (csrc/host.cpp) under the host compiler's
address and undefined-behaviour sanitizers: a randomized driver (tests/native/host_check.cpp)
feeds the validators and planners hundreds of thousands of argument sets, including
out-of-range sizes and misaligned or NULL pointers, and checks the plans' invariants."""
import os
import shutil
import subprocess

import pytest

from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "bit_kv_cache_kvq_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs the host C++ compiler")
def test_host_code_under_sanitizers(tmp_path):
    exe = tmp_path / "host_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "host.cpp"), os.path.join(ROOT, "tests", "native", "host_check.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.startswith("host_check ok"), r.stdout
