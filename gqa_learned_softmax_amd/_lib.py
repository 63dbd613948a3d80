"""ctypes binding of libsinkattn (include/sinkattn.h). Argument marshalling only.

Torch supplies device memory and the current HIP stream; every step of the computation runs in
the library's HIP kernels. There is no fallback: if ``libsinkattn.so`` is missing, importing this
module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

# The library this module binds. SINKATTN_LIBRARY names another build of the same C ABI instead
# (a debug build of the kernels, or the host-only build used to check the ABI layer without a GPU).
DEFAULT_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsinkattn.so")
LIB_PATH = os.environ.get("SINKATTN_LIBRARY") or DEFAULT_LIB_PATH

# sinkattn_status
OK = 0
ERR_NULL = 1
ERR_DTYPE = 2
ERR_SHAPE = 3
ERR_LAYOUT = 4
ERR_UNSUPPORTED = 5
ERR_LAUNCH = 6

# sinkattn_dtype
F32 = 0
BF16 = 1
I32 = 2
FP8_E4M3 = 3
_DTYPE_CODE = {torch.float32: F32, torch.bfloat16: BF16, torch.int32: I32, torch.float8_e4m3fn: FP8_E4M3}
_UNKNOWN_DTYPE = 99  # the library rejects it with SINKATTN_ERR_DTYPE


class SinkAttnError(RuntimeError):
    """A non-OK status from libsinkattn."""

    def __init__(self, status: int, message: str):
        super().__init__(f"sinkattn error {status}: {message}")
        self.status = status
        self.message = message


class Tensor(ctypes.Structure):
    """``sinkattn_tensor``."""

    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int),
        ("ndim", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 4),
        ("stride", ctypes.c_int64 * 4),
    ]


_P = ctypes.POINTER(Tensor)


class Launch(ctypes.Structure):
    """``sinkattn_launch``."""

    _fields_ = [("kernel", ctypes.c_char * 96), ("grid", ctypes.c_int64), ("block", ctypes.c_int32)]


_L = ctypes.POINTER(Launch)
_IP = ctypes.POINTER(ctypes.c_int)

# sinkattn_plan_form
PLAN_DECODE_SPLIT = 0
PLAN_DECODE = 1

EXPORTS = {
    "sinkattn_prefill": ([_P, _P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_int, _P, ctypes.c_void_p],
                         ctypes.c_int),
    "sinkattn_prefill_split": ([_P, _P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_int, ctypes.c_int, _P, _P, _P,
                                ctypes.c_void_p], ctypes.c_int),
    "sinkattn_decode_split": ([_P, _P, _P, _P, _P, ctypes.c_int, ctypes.c_float, _P, _P, _P,
                               ctypes.c_void_p], ctypes.c_int),
    "sinkattn_decode_multi_split": ([_P, _P, _P, _P, _P, ctypes.c_int, ctypes.c_float, _P, _P, _P,
                                     ctypes.c_void_p], ctypes.c_int),
    "sinkattn_decode_merge": ([_P, _P, _P, ctypes.c_int, _P, _P, ctypes.c_void_p], ctypes.c_int),
    "sinkattn_decode": ([_P, _P, _P, _P, _P, ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                         ctypes.c_size_t, _P, _P, ctypes.c_void_p], ctypes.c_int),
    "sinkattn_decode_multi": ([_P, _P, _P, _P, _P, ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                               ctypes.c_size_t, _P, _P, ctypes.c_void_p], ctypes.c_int),
    "sinkattn_decode_static": ([_P, _P, _P, _P, _P, ctypes.c_int, ctypes.c_float, _P, _P, ctypes.c_void_p],
                               ctypes.c_int),
    "sinkattn_decode_workspace_size": ([ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int],
                                       ctypes.c_size_t),
    "sinkattn_decode_workspace_counter_bytes": ([ctypes.c_int64, ctypes.c_int64], ctypes.c_size_t),
    "sinkattn_moe_topk_softmax": ([_P, ctypes.c_int, ctypes.c_int, _P, _P, ctypes.c_void_p], ctypes.c_int),
    "sinkattn_linear_bias": ([_P, _P, _P, _P, ctypes.c_void_p], ctypes.c_int),
    "sinkattn_linear_fp8_block_scaled": ([_P, _P, _P, _P, _P, _P, ctypes.c_void_p], ctypes.c_int),
    "sinkattn_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "sinkattn_plan_decode": ([_P, _P, _P, _P, _P, ctypes.c_int, ctypes.c_float, ctypes.c_int, _L, _IP],
                             ctypes.c_int),
    "sinkattn_plan_prefill": ([_P, _P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_int, ctypes.c_int, _L, _IP],
                              ctypes.c_int),
    "sinkattn_last_error": ([], ctypes.c_char_p),
    "sinkattn_version": ([], ctypes.c_int),
}


def load(path: str) -> ctypes.CDLL:
    """Loads a build of the C ABI at ``path`` and declares every exported function's types."""
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python gqa_learned_softmax_amd/build.py` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    for name, (argtypes, restype) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = restype
    return lib


lib = load(LIB_PATH)


def describe(t: torch.Tensor | None) -> Tensor | None:
    """Descriptor for a tensor view (no copy)."""
    if t is None:
        return None
    if t.dim() > 4:
        raise SinkAttnError(ERR_SHAPE, f"rank {t.dim()} > 4")
    d = Tensor()
    d.data = t.data_ptr() if t.numel() > 0 else None
    d.dtype = _DTYPE_CODE.get(t.dtype, _UNKNOWN_DTYPE)
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def ref(d: Tensor | None):
    return ctypes.byref(d) if d is not None else None


def check(status: int) -> None:
    if status != OK:
        msg = lib.sinkattn_last_error().decode() or lib.sinkattn_status_string(status).decode()
        raise SinkAttnError(status, msg)


def require_device(*tensors) -> torch.device:
    """All tensors must live on one GPU: the kernels dereference their pointers on the device."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise SinkAttnError(ERR_LAYOUT, "tensors must be on a GPU (HIP) device")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise SinkAttnError(ERR_LAYOUT, "tensors must be on the same device")
    return dev


def stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream
