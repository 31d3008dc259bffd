"""Build libhe.so (HIP kernels + C++ runtime) for gfx950 with hipcc.

    python -m transformer_decode_amd.build        # or __graft_entry__.build()

Objects go to ``_build/`` at the repository root; the shared library is written
next to this file (``transformer_decode_amd/libhe.so``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libhe.so")

ARCH = "gfx950"
SOURCES = ["k_elem.hip", "k_gemm.hip", "k_gemv.hip", "k_attn.hip", "k_fp8.hip", "k_static.hip", "he_api.cpp"]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libhe)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    flags_txt = " ".join(COMMON[:4] + DEVICE_FLAGS)
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, f'-DHE_BUILD_FLAGS="{flags_txt}"', "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libhe_asan.so")


def asan_runtime() -> str:
    """The shared AddressSanitizer runtime of the ROCm clang (to preload into a host process)."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        import glob
        hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        if not hits:
            raise RuntimeError("AddressSanitizer runtime not found")
        path = hits[0]
    return path


def build_asan(verbose: bool = True) -> str:
    """libhe with the host runtime (he_api.cpp) built under AddressSanitizer, for the
    host-side tests (HE_FLAG_VALIDATE_ONLY).  The sanitizer applies to host code only
    (each -fsanitize sits after -Xarch_host); the kernels are the normal build's objects."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    heads = [os.path.join(CSRC, h) for h in ("common.h", "kernels.h")] + [os.path.join(INCLUDE, "he.h")]
    newest_head = max(os.path.getmtime(h) for h in heads)
    for s in SOURCES:                     # the kernels' objects of the normal build, made if stale
        o = os.path.join(BUILD, s + ".o")
        if s != "he_api.cpp" and (not os.path.exists(o) or os.path.getmtime(o) <
                                  max(newest_head, os.path.getmtime(os.path.join(CSRC, s)))):
            os.makedirs(BUILD, exist_ok=True)
            _compile(s)
    obj = os.path.join(ASAN_DIR, "he_api.cpp.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *san, "-c", os.path.join(CSRC, "he_api.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling he_api.cpp with ASan failed:\n{' '.join(cmd)}\n{r.stderr}")
    objs = [os.path.join(BUILD, s + ".o") for s in SOURCES if s != "he_api.cpp"] + [obj]
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Xarch_host", "-fsanitize=address",
           "-shared-libasan", *objs, "-o", ASAN_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking the ASan library failed:\n{' '.join(cmd)}\n{r.stderr}")
    if verbose:
        print(f"built {ASAN_LIB}")
    return ASAN_LIB


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libhe.so failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
