"""Build libpagedkv.so (the C-ABI library of gfx950 kernels) in-tree with hipcc.

    python -m paged_kv_cache_09_amd.build            # build
    python -m paged_kv_cache_09_amd.build --asm      # also keep AMD GCN assembly in _build/

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled, and linked into paged_kv_cache_09_amd/libpagedkv.so.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")
SOURCES = ["api.hip", "append.hip", "copy.hip", "decode_g1.hip", "decode_mfma.hip",
           "reduce.hip"]
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, asm: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if asm:
        cmd += ["-save-temps=obj"]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=BUILD)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    errs = [ln for ln in r.stderr.splitlines()
            if "packed-fp32-ops" not in ln and ln.strip() and "warning" in ln]
    for ln in errs:
        sys.stderr.write(ln + "\n")
    return obj


# A plain-C program that drives the library through include/paged_kv.h only (no
# Python, no torch); the GPU tests run it.
C_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi_check.c")
C_CHECK_BIN = os.path.join(ROOT, "tests", "c_abi_check")


def build_c_check() -> str:
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler for the C-ABI check")
    tmp = C_CHECK_BIN + ".tmp%d" % os.getpid()
    cmd = [cc, "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(rocm, 'include')}", f"-I{os.path.join(ROOT, 'include')}",
           C_CHECK_SRC, "-o", tmp, f"-L{PKG}", "-lpagedkv", f"-L{os.path.join(rocm, 'lib')}",
           "-lamdhip64", "-lm", "-Wl,-rpath,$ORIGIN/../paged_kv_cache_09_amd",
           f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("building the C-ABI check failed")
    os.replace(tmp, C_CHECK_BIN)
    return C_CHECK_BIN


def build(asm: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, asm), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True, capture_output=True, cwd=BUILD)
    os.replace(tmp, LIB)
    build_c_check()
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", action="store_true", help="keep device assembly under _build/")
    args = ap.parse_args()
    print(build(asm=args.asm))


if __name__ == "__main__":
    main()
