"""Build libqsa.so (the HIP kernels and the C-ABI) in-tree for gfx950.

    python -m block_sparse_long_amd.build        # or build() from Python

Every source under csrc/ is compiled with hipcc for gfx950 only, in parallel,
into _build/, and linked into block_sparse_long_amd/libqsa.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libqsa.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "pool.hip", "score.hip", "select.hip", "attn.hip", "attn_mfma.hip", "score_fused.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def _flags() -> list:
    return ["-x", "hip", "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
            # packed fp32 VALU instructions stay off: ordinary float code is
            # compiled to plain VALU ops only
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + _flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile and link libqsa.so; returns its path.  Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    workers = min(len(SOURCES), max(1, (os.cpu_count() or 2) // 2))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}"] + objs + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
