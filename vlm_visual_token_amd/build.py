"""Build libivc.so (the connector's C-ABI library) in-tree with hipcc for gfx950.

    python -m vlm_visual_token_amd.build

Objects go to ``_build/``; the library lands next to this file.  Every HIP
source is compiled with packed-fp32 code generation turned off.

Two host-only debug builds sit beside it:

* ``libivc_index_check.so`` (g++, ``IVC_DEBUG``): the kernels' index math
  (``csrc/index_math.h``) with bounds checks, walked on the CPU by the tests;
* ``build_sanitized()``: the same library with AddressSanitizer and
  UndefinedBehaviorSanitizer on its host code only (the GPU code is built as
  usual), plus the index self-test executable, for the CPU tests of the
  host-side validation paths.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libivc.so")
INDEX_LIB = os.path.join(PKG, "libivc_index_check.so")
SAN_DIR = os.path.join(BUILD, "san")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build_index_check() -> str:
    """The index math with bounds checks, as a host shared library."""
    tmp = INDEX_LIB + ".tmp"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-DIVC_DEBUG", "-shared", "-fPIC", "-I", CSRC,
           os.path.join(CSRC, "index_check.cpp"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed for index_check.cpp:\n{r.stderr}")
    os.replace(tmp, INDEX_LIB)
    return INDEX_LIB


def _san_compile(src: str) -> str:
    obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
    # sanitizers on the host pass only: the GPU code is built exactly as usual
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    cmd = [HIPCC, *FLAGS, "-g", *san, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc (sanitized host) failed for {src}:\n{r.stderr}")
    return obj


def build_sanitized() -> dict:
    """Host-sanitized libivc.so and the sanitized index self-test, under
    _build/san/.  Returns their paths and the runtime a Python process must
    preload to load the library."""
    os.makedirs(SAN_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_san_compile, srcs))
    lib = os.path.join(SAN_DIR, "libivc.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan", *san, *objs,
           "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    exe = os.path.join(SAN_DIR, "index_selftest")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-DIVC_INDEX_CHECK_MAIN",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-I", CSRC,
           os.path.join(CSRC, "index_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed for the index self-test:\n{r.stderr}")
    rt = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True).stdout.strip()
    return {"lib": lib, "selftest": exe, "asan_runtime": rt}


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    build_index_check()
    if verbose:
        print(f"built {LIB} and {INDEX_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
