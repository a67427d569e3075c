"""Build libfd.so (the HIP library behind include/fd.h) for gfx950 in-tree.

Every source is compiled by hipcc with packed-fp32 instructions disabled
(they are not emitted by hand either), objects go to ``_build/`` at the
repository root, and the shared library lands next to this file. Always
recompiles when called.

    python -m decode_attention_09_amd.build
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
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfd.so")
ARCH = "gfx950"

SOURCES = ["fd_split_f32.hip", "fd_split_f16.hip", "fd_split_bf16.hip", "fd_combine.hip",
           "fd_api.hip"]

FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # the split kernels' first two arguments (cu_seqlens_k, batch) arrive
         # preloaded in SGPRs
         "-mllvm", "-amdgpu-kernarg-preload-count=2",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libfd)")


def _flags():
    # FD_HIPCC_FLAGS: extra hipcc flags (e.g. -DFD_PREFETCH_TILES_VALU=2)
    return FLAGS + os.environ.get("FD_HIPCC_FLAGS", "").split()


def _compile(src: str, obj_dir: str = OBJ) -> str:
    obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, lib_path: str = LIB, obj_dir: str = OBJ) -> str:
    os.makedirs(obj_dir, exist_ok=True)
    workers = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(lambda src: _compile(src, obj_dir), SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
