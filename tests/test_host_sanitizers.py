"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

A second copy of libmqa.so is built into a temporary folder with both sanitizers on the
host code only (the GPU code is compiled as usual), a C++ driver (host_abi_check.cpp)
calls every entry point with the rejected and edge-case arguments of the Python ABI
tests, and the run must end cleanly: every status as documented in include/mqa.h, no
sanitizer report, no leak. Nothing reaches a GPU (each call is rejected, is a no-op or
is a size query), so this runs without one.
"""
import os
import shutil
import subprocess

import pytest

from fp8_paged_mqa_amd import build as mqa_build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(not os.path.exists(mqa_build.HIPCC), reason="hipcc not installed")
def test_c_abi_host_checks_under_asan_and_ubsan(tmp_path):
    lib = mqa_build.build(out_dir=str(tmp_path), sanitize=True)
    exe = str(tmp_path / "host_abi_check")
    cmd = [mqa_build.HIPCC, "-std=c++17", "-g", "-Wall", f"-I{os.path.join(ROOT, 'include')}",
           *mqa_build.SANITIZE, os.path.join(HERE, "host_abi_check.cpp"),
           f"-L{tmp_path}", "-lmqa", f"-Wl,-rpath,{tmp_path}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in out and "LeakSanitizer" not in out and "runtime error" not in out, out
    assert out.strip().splitlines()[-1].startswith("ok:"), out
    assert os.path.getsize(lib) > 0
    shutil.rmtree(tmp_path / "obj", ignore_errors=True)
