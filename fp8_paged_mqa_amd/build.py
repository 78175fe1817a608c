"""Builds libmqa.so (HIP kernels for gfx950 + the C-ABI host layer) in-tree.

    python -m fp8_paged_mqa_amd.build

Every call recompiles. Objects go to fp8_paged_mqa_amd/_build/, the library to
fp8_paged_mqa_amd/libmqa.so.

build(out_dir=D, sanitize=True) builds a second copy into D with AddressSanitizer and
UndefinedBehaviorSanitizer on the host code only (the host checks of the C ABI); the GPU
code is compiled as usual. That copy is for host-side test drivers, never for loading
into Python.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmqa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
# Packed fp32 VALU ops (v_pk_*_f32) are kept out of the generated code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]
# Host-only sanitizers: each -fsanitize= is preceded by -Xarch_host so that no GPU code is
# instrumented.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False, out_dir: str | None = None, sanitize: bool = False) -> str:
    """Compiles every source and links libmqa.so; returns the library's path. With out_dir
    the objects and the library go there instead of the package."""
    obj_dir = OBJ if out_dir is None else os.path.join(out_dir, "obj")
    lib = LIB if out_dir is None else os.path.join(out_dir, "libmqa.so")
    extra = SANITIZE if sanitize else []
    os.makedirs(obj_dir, exist_ok=True)
    jobs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
        jobs.append([HIPCC, *COMMON, *DEVICE, *extra, "-c", src, "-o", obj])
    for src in sorted(glob.glob(os.path.join(CSRC, "*.cpp"))):
        obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
        jobs.append([HIPCC, *COMMON, *extra, "-c", src, "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for r in ex.map(_run, jobs):
            if verbose and (r.stdout or r.stderr):
                print(r.stdout, r.stderr, file=sys.stderr)
    objs = [j[-1] for j in jobs]
    tmp = lib + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *extra, *objs, "-o", tmp])
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
