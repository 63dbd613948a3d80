"""The C-ABI layer (api.cpp) built for the host alone and run under AddressSanitizer and
UndefinedBehaviorSanitizer, with stub launchers (tests/host/stub_launch.cpp) in place of the HIP
kernel files: no GPU and no HIP runtime involved.

In a child process (the sanitizer runtime must be loaded first, hence LD_PRELOAD) this runs
  * tests/host/accepted_calls.py: accepted calls and what they hand each launcher (grids, chunk
    size, single-launch decision, workspace carving, prefill grid bound, plan queries);
  * tests/test_abi.py: every rejection and empty call of the ABI suite, now under the sanitizers.
Any sanitizer report aborts the child.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gqa_learned_softmax_amd", "csrc")
OUT_DIR = os.path.join(ROOT, "_build", "host")
STUB_LIB = os.path.join(OUT_DIR, "libsinkattn_hoststub.so")
ROCM_INCLUDE = "/opt/rocm/include"


def _sanitizer_runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def build_host_stub():
    """g++ build of api.cpp + the stub launchers with ASan and UBSan (host code only)."""
    os.makedirs(OUT_DIR, exist_ok=True)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INCLUDE}", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "api.cpp"), os.path.join(ROOT, "tests", "host", "stub_launch.cpp"),
           "-o", STUB_LIB]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return STUB_LIB


@pytest.fixture(scope="module")
def stub_lib():
    if shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("needs g++ and the ROCm headers")
    if _sanitizer_runtime("libasan.so") is None:
        pytest.skip("needs g++'s AddressSanitizer runtime")
    return build_host_stub()


def test_abi_layer_under_address_and_undefined_behaviour_sanitizers(stub_lib):
    env = dict(os.environ)
    env.update({
        "SINKATTN_LIBRARY": stub_lib,
        "LD_PRELOAD": _sanitizer_runtime("libasan.so"),
        # Python itself keeps objects alive until exit: leak reports would only show those.
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        "PYTHONDONTWRITEBYTECODE": "1",
    })
    # -s: a sanitizer report goes to stderr as it happens, not into pytest's capture.
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "host", "accepted_calls.py"), os.path.join(ROOT, "tests", "test_abi.py")]
    res = subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT, env=env, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-6000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert " passed" in out and "skipped" not in out.split("\n")[-2], out[-2000:]
