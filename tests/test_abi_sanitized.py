"""The library's host-side code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

The library sources are compiled as in the normal build, with the sanitizers on
the host pass only (each -fsanitize= right after -Xarch_host, so no device
code is instrumented), and linked into tests/abi_host_driver.cpp.  The
driver calls every entry point over shapes up to and past each limit:
workspace sizes, rejected calls and status strings.  None of its calls
reaches a kernel launch, so no GPU is needed.  Any sanitizer report aborts
the driver, and so fails the test.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from long_context_sparse_routing_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
SAN = ["-Xarch_host", "-fsanitize=address",
       "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")
def test_host_code_under_asan_and_ubsan(tmp_path):
    base = [B.HIPCC, f"--offload-arch={B.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", *SAN,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(B.ROOT, "include")]

    def compile_one(src):
        obj = str(tmp_path / src.replace(".hip", ".o"))
        cmd = [*base, *B.EXTRA.get(src, []), "-c", os.path.join(B.CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-3000:]
        return obj

    with ThreadPoolExecutor(max_workers=len(B.SOURCES)) as ex:
        objs = list(ex.map(compile_one, B.SOURCES))
    exe = str(tmp_path / "abi_host_driver")
    cmd = [*base, "-x", "c++", os.path.join(HERE, "abi_host_driver.cpp"), "-x", "none", *objs,
           "-o", exe, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, (res.stdout + res.stderr)[-4000:]
    assert "host ABI paths clean" in res.stdout
