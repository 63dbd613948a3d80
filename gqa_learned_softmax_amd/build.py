"""Builds libsinkattn.so (the C-ABI HIP library) in-tree with hipcc for gfx950.

Usage: ``python gqa_learned_softmax_amd/build.py`` (or ``__graft_entry__.build()``). Sources are
compiled to objects in parallel, then linked into ``gqa_learned_softmax_amd/libsinkattn.so``; the
measurement kernels (``csrc/ceilings.hip``) go into ``libsinkattn_ceilings.so`` beside it.
Every call recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libsinkattn.so")

SOURCES = ["api.cpp", "decode_split.hip", "decode_merge.hip", "prefill.hip", "moe_topk.hip", "gemm.hip",
           "static_workspace.hip"]
CEILING_SOURCES = ["ceilings.hip"]
CEILINGS_LIB_PATH = os.path.join(PKG_DIR, "libsinkattn_ceilings.so")

ARCH = "gfx950"
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # Packed fp32 vector ops stay off: the kernels use scalar fp32 VALU math only.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libsinkattn")


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, path: str) -> None:
    tmp = path + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, path)


def build(extra_flags=(), verbose: bool = False) -> str:
    """Compile every source and link libsinkattn.so and libsinkattn_ceilings.so; returns the
    path of libsinkattn.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = SOURCES + CEILING_SOURCES
    with ThreadPoolExecutor(max_workers=min(4, len(sources))) as pool:
        objs = list(pool.map(lambda s: _compile(s, list(extra_flags)), sources))
    _link(objs[:len(SOURCES)], LIB_PATH)
    _link(objs[len(SOURCES):], CEILINGS_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {CEILINGS_LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(extra_flags=sys.argv[1:], verbose=True)
