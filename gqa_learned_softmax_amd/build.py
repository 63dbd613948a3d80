"""Builds libsinkattn.so (the C-ABI HIP library) in-tree with hipcc for gfx950.

Usage: ``python gqa_learned_softmax_amd/build.py`` (or ``__graft_entry__.build()``). Sources are
compiled to objects in parallel, then linked into ``gqa_learned_softmax_amd/libsinkattn.so``; the
measurement kernels (``csrc/ceilings.hip``) go into ``libsinkattn_ceilings.so`` beside it, and the
debug builds of the attention kernels (poisoned LDS, two deliberate mistakes in the sink rule; see
``csrc/device_common.h``) into ``libsinkattn_<variant>.so``, which only tests load.
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

# Debug builds: the same library with one switch of csrc/device_common.h defined. Only the kernel
# files that read the switches are compiled again; the rest are linked from the main build.
DEBUG_VARIANTS = {
    "poison_lds": ["-DSINKATTN_POISON_LDS"],
    "mutate_sink_every_chunk": ["-DSINKATTN_MUTATE_SINK_EVERY_CHUNK"],
    "mutate_d0_zero": ["-DSINKATTN_MUTATE_D0_ZERO"],
}
VARIANT_SOURCES = ["decode_split.hip", "prefill.hip"]


def variant_path(name: str) -> str:
    return os.path.join(PKG_DIR, f"libsinkattn_{name}.so")

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


def _compile(src: str, extra, obj_dir: str = BUILD_DIR) -> str:
    os.makedirs(obj_dir, exist_ok=True)
    obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
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
    """Compile every source and link libsinkattn.so, libsinkattn_ceilings.so and the debug
    variants; returns the path of libsinkattn.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = list(extra_flags)
    jobs = [(src, extra, BUILD_DIR) for src in SOURCES + CEILING_SOURCES]
    for name, flags in DEBUG_VARIANTS.items():
        jobs += [(src, extra + flags, os.path.join(BUILD_DIR, name)) for src in VARIANT_SOURCES]
    workers = max(1, min(8, os.cpu_count() or 1, len(jobs)))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        objs = list(pool.map(lambda job: _compile(*job), jobs))
    main = dict(zip(SOURCES, objs[:len(SOURCES)]))
    _link([main[s] for s in SOURCES], LIB_PATH)
    _link(objs[len(SOURCES):len(SOURCES) + len(CEILING_SOURCES)], CEILINGS_LIB_PATH)
    pos = len(SOURCES) + len(CEILING_SOURCES)
    for name in DEBUG_VARIANTS:
        swapped = dict(main)
        for src in VARIANT_SOURCES:
            swapped[src] = objs[pos]
            pos += 1
        _link([swapped[s] for s in SOURCES], variant_path(name))
    if verbose:
        print(f"built {LIB_PATH}, {CEILINGS_LIB_PATH} and {len(DEBUG_VARIANTS)} debug variants")
    return LIB_PATH


if __name__ == "__main__":
    build(extra_flags=sys.argv[1:], verbose=True)
