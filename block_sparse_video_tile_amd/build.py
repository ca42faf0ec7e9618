"""Build libvsa_amd.so in-tree with hipcc for gfx950.

Usage: python -m block_sparse_video_tile_amd.build [--asan]
(or build_library() / build_asan_library() from Python).
Every source is compiled in parallel to an object file under _build/, then
linked into block_sparse_video_tile_amd/libvsa_amd.so.  --asan also links
_build/asan/libvsa_amd_asan.so, whose host code is built with
AddressSanitizer, for the host-only ABI tests.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libvsa_amd.so")
ARCH = "gfx950"

SOURCES = ["vsa_api.cpp", "gather_scatter.hip", "score_topk.hip", "attention.hip", "coarse.hip", "backward.hip",
           "microbench.hip"]

# Packed fp32 VALU ops are kept out of the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
                f"-I{INCLUDE}", f"-I{CSRC}"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm under /opt/rocm)")


def _compile(src: str, hipcc: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip", f"--offload-arch={ARCH}", *DEVICE_FLAGS]
    else:
        cmd[1:1] = ["-D__HIP_PLATFORM_AMD__"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build_library(verbose: bool = False) -> str:
    """Compile every HIP/C++ source for gfx950 and link the shared library."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


ASAN_LIB_PATH = os.path.join(BUILD_DIR, "asan", "libvsa_amd_asan.so")


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (for LD_PRELOAD)."""
    res = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the shared AddressSanitizer runtime was not found")
    return path


def build_asan_library(verbose: bool = False) -> str:
    """The same library with its host code (the planner and argument checks,
    vsa_api.cpp) built with AddressSanitizer, for host-only tests; the
    device objects are the regular ones.  Never loaded on a GPU path."""
    hipcc = _hipcc()
    out_dir = os.path.dirname(ASAN_LIB_PATH)
    os.makedirs(out_dir, exist_ok=True)
    asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-shared-libasan"]
    api_obj = os.path.join(out_dir, "vsa_api.cpp.o")
    cmd = [hipcc, "-D__HIP_PLATFORM_AMD__", *COMMON_FLAGS, "-g", *asan, "-c",
           os.path.join(CSRC, "vsa_api.cpp"), "-o", api_obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    dev_objs = [os.path.join(BUILD_DIR, src + ".o") for src in SOURCES if src.endswith(".hip")]
    missing = [o for o in dev_objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"build the library first (missing {missing})")
    tmp = ASAN_LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *asan, "-o", tmp, api_obj,
           *dev_objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, ASAN_LIB_PATH)
    if verbose:
        print(f"built {ASAN_LIB_PATH}")
    return ASAN_LIB_PATH


if __name__ == "__main__":
    build_library(verbose=True)
    if "--asan" in sys.argv[1:]:
        build_asan_library(verbose=True)
    sys.exit(0)
