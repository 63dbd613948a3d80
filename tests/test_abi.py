"""C-ABI checks that need no GPU: the library loads, exports every function include/sinkattn.h
declares, and rejects every malformed call on the host, before any HIP call.

Descriptors here carry fake (but aligned, disjoint) device addresses: validation never
dereferences them, and every call below is rejected before a launch could happen. The only
accepted calls are the empty ones (Tq = 0, B = 0), which launch nothing by contract.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from gqa_learned_softmax_amd import _lib
from gqa_learned_softmax_amd._lib import BF16, F32, I32, Tensor

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "sinkattn.h")

_next_addr = [1 << 40]


def T(shape, dtype=BF16, strides=None, addr=None):
    d = Tensor()
    if addr is None:
        addr = _next_addr[0]
        _next_addr[0] += 1 << 32  # every tensor in its own 4 GiB window: no accidental overlap
    d.data = addr
    d.dtype = dtype
    d.ndim = len(shape)
    if strides is None:
        strides, acc = [], 1
        for n in reversed(shape):
            strides.insert(0, acc)
            acc *= n
    for i, (n, s) in enumerate(zip(shape, strides)):
        d.shape[i] = n
        d.stride[i] = s
    return d


def R(d):
    return ctypes.byref(d) if d is not None else None


def last_error():
    return _lib.lib.sinkattn_last_error().decode()


# ----------------------------------------------------------------------------- exports
def test_every_declared_function_is_exported():
    text = open(HEADER).read()
    names = set(re.findall(r"^\s*(?:const\s+char\s*\*|sinkattn_status|int|size_t)\s+(sinkattn_\w+)\s*\(",
                           text, flags=re.M))
    assert {"sinkattn_prefill", "sinkattn_decode_split", "sinkattn_decode_merge"} <= names
    for name in names:
        assert hasattr(_lib.lib, name), name
    assert names == set(_lib.EXPORTS)


CEILINGS_HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "sinkattn_ceilings.h")
CEILINGS_LIB = os.path.join(os.path.dirname(_lib.DEFAULT_LIB_PATH), "libsinkattn_ceilings.so")


def test_ceilings_library_exports_its_header_and_rejects_bad_arguments():
    """The measurement library loads, exports what include/sinkattn_ceilings.h declares, and
    rejects invalid arguments on the host (return 1) without launching anything."""
    text = open(CEILINGS_HEADER).read()
    names = set(re.findall(r"^\s*(?:int|double)\s+(sinkattn_ceiling_\w+)\s*\(", text, flags=re.M))
    assert names == {"sinkattn_ceiling_stream_read", "sinkattn_ceiling_stream_read_slices", "sinkattn_ceiling_mfma_bf16",
                     "sinkattn_ceiling_mfma_bf16_flop", "sinkattn_ceiling_mfma_bf16_random",
                     "sinkattn_ceiling_mfma_bf16_random_flop", "sinkattn_ceiling_issue"}
    lib = ctypes.CDLL(CEILINGS_LIB)
    for name in names:
        assert hasattr(lib, name), name
    lib.sinkattn_ceiling_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int,
                                                 ctypes.c_void_p, ctypes.c_void_p]
    lib.sinkattn_ceiling_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.sinkattn_ceiling_mfma_bf16_flop.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.sinkattn_ceiling_mfma_bf16_flop.restype = ctypes.c_double
    fake = 1 << 40
    assert lib.sinkattn_ceiling_stream_read(None, 1 << 20, 64, fake, None) == 1
    assert lib.sinkattn_ceiling_stream_read(fake, (1 << 20) + 8, 64, fake, None) == 1  # not whole 16 B
    assert lib.sinkattn_ceiling_stream_read(fake + 8, 1 << 20, 64, fake, None) == 1    # misaligned
    assert lib.sinkattn_ceiling_stream_read(fake, 1 << 20, 0, fake, None) == 1
    assert lib.sinkattn_ceiling_mfma_bf16(0, 10, fake, None) == 1
    assert lib.sinkattn_ceiling_mfma_bf16(8, 0, fake, None) == 1
    lib.sinkattn_ceiling_issue.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p]
    assert lib.sinkattn_ceiling_issue(8, 8, 10, fake, fake, None) == 1   # no such kind
    assert lib.sinkattn_ceiling_issue(-1, 8, 10, fake, fake, None) == 1
    lib.sinkattn_ceiling_stream_read_slices.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                                        ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    sl = lib.sinkattn_ceiling_stream_read_slices
    assert sl(None, fake, 8, 8, 1024, 1024, fake, None) == 1
    assert sl(fake, fake + 8, 8, 8, 1024, 1024, fake, None) == 1     # misaligned V
    assert sl(fake, fake, 8, 8, 1024, 1000, fake, None) == 1         # rows not whole 256-byte slices
    assert sl(fake, fake, 0, 8, 1024, 1024, fake, None) == 1
    assert sl(fake, fake, 8, 8, 0, 1024, fake, None) == 1
    assert sl(fake, fake, 8, 8, 1024, 1024, None, None) == 1
    assert lib.sinkattn_ceiling_issue(0, 0, 10, fake, fake, None) == 1
    assert lib.sinkattn_ceiling_issue(0, 8, 0, fake, fake, None) == 1
    assert lib.sinkattn_ceiling_issue(0, 8, 10, None, fake, None) == 1
    # 4 waves x 4 MFMAs of 32 x 32 x 16 x 2 flop per block and iteration.
    assert lib.sinkattn_ceiling_mfma_bf16_flop(3, 5) == 3 * 5 * 4 * 4 * 32 * 32 * 16 * 2
    lib.sinkattn_ceiling_mfma_bf16_random.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.sinkattn_ceiling_mfma_bf16_random_flop.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.sinkattn_ceiling_mfma_bf16_random_flop.restype = ctypes.c_double
    assert lib.sinkattn_ceiling_mfma_bf16_random(0, 10, fake, None) == 1
    assert lib.sinkattn_ceiling_mfma_bf16_random(8, 0, fake, None) == 1
    assert lib.sinkattn_ceiling_mfma_bf16_random(8, 10, None, None) == 1
    assert lib.sinkattn_ceiling_mfma_bf16_random_flop(3, 5) == 3 * 5 * 4 * 8 * 32 * 32 * 16 * 2


def test_version_and_status_strings():
    text = open(HEADER).read()
    version = int(re.search(r"#define SINKATTN_VERSION (\d+)", text).group(1))
    assert _lib.lib.sinkattn_version() == version
    for code in range(7):
        s = _lib.lib.sinkattn_status_string(code).decode()
        assert s and s != "unknown status"
    assert _lib.lib.sinkattn_status_string(123).decode() == "unknown status"


# ----------------------------------------------------------------------------- prefill
def prefill_args(tq=16, hq=8, hkv=2, dim=64, b=1, dtype=BF16, out_dtype=None):
    return dict(
        q=T([tq, hq, dim], dtype), k=T([tq, hkv, dim], dtype), v=T([tq, hkv, dim], dtype),
        sinks=T([hq], F32), cu_q=T([b + 1], I32), cu_k=T([b + 1], I32),
        out=T([tq, hq, dim], out_dtype if out_dtype is not None else dtype), scale=0.125, causal=1)


def call_prefill(a):
    return _lib.lib.sinkattn_prefill(R(a["q"]), R(a["k"]), R(a["v"]), R(a["sinks"]), R(a["cu_q"]),
                                     R(a["cu_k"]), a["scale"], a["causal"], R(a["out"]), None)


def test_prefill_empty_batch_is_ok_and_launches_nothing():
    assert call_prefill(prefill_args(tq=0)) == _lib.OK
    assert call_prefill(prefill_args(tq=0, b=0)) == _lib.OK


def _mut(a, **kw):
    a = dict(a)
    a.update(kw)
    return a


PREFILL_CASES = [
    ("q_null", lambda a: _mut(a, q=None), _lib.ERR_NULL),
    ("out_null", lambda a: _mut(a, out=None), _lib.ERR_NULL),
    ("sinks_null", lambda a: _mut(a, sinks=None), _lib.ERR_NULL),
    ("q_data_null", lambda a: _mut(a, q=T([16, 8, 64], addr=0)), _lib.ERR_NULL),
    ("k_dtype_mismatch", lambda a: _mut(a, k=T([16, 2, 64], F32)), _lib.ERR_DTYPE),
    ("q_int", lambda a: _mut(a, q=T([16, 8, 64], I32)), _lib.ERR_DTYPE),
    ("unknown_dtype", lambda a: _mut(a, v=T([16, 2, 64], 7)), _lib.ERR_DTYPE),
    ("sinks_bf16", lambda a: _mut(a, sinks=T([8], BF16)), _lib.ERR_DTYPE),
    ("cu_f32", lambda a: _mut(a, cu_q=T([2], F32)), _lib.ERR_DTYPE),
    ("q_rank2", lambda a: _mut(a, q=T([16, 512])), _lib.ERR_SHAPE),
    ("heads_not_multiple", lambda a: _mut(a, q=T([16, 6, 64]), out=T([16, 6, 64]), sinks=T([6], F32),
                                          k=T([16, 4, 64]), v=T([16, 4, 64])), _lib.ERR_SHAPE),
    ("out_shape", lambda a: _mut(a, out=T([16, 4, 64])), _lib.ERR_SHAPE),
    ("v_shape", lambda a: _mut(a, v=T([15, 2, 64])), _lib.ERR_SHAPE),
    ("k_dim", lambda a: _mut(a, k=T([16, 2, 32]), v=T([16, 2, 32])), _lib.ERR_SHAPE),
    ("sinks_len", lambda a: _mut(a, sinks=T([7], F32)), _lib.ERR_SHAPE),
    ("cu_len_mismatch", lambda a: _mut(a, cu_k=T([3], I32)), _lib.ERR_SHAPE),
    ("cu_empty", lambda a: _mut(a, cu_q=T([0], I32), cu_k=T([0], I32)), _lib.ERR_SHAPE),
    ("scale_zero", lambda a: _mut(a, scale=0.0), _lib.ERR_SHAPE),
    ("scale_negative", lambda a: _mut(a, scale=-0.125), _lib.ERR_SHAPE),
    ("scale_nan", lambda a: _mut(a, scale=float("nan")), _lib.ERR_SHAPE),
    ("scale_inf", lambda a: _mut(a, scale=float("inf")), _lib.ERR_SHAPE),
    ("head_dim_128", lambda a: prefill_args(dim=128), _lib.ERR_UNSUPPORTED),
    ("group_3", lambda a: prefill_args(hq=6, hkv=2), _lib.ERR_UNSUPPORTED),
    ("q_misaligned", lambda a: _mut(a, q=T([16, 8, 64], addr=(3 << 44) + 2)), _lib.ERR_LAYOUT),
    ("q_inner_stride", lambda a: _mut(a, q=T([16, 8, 64], strides=[1024, 128, 2])), _lib.ERR_LAYOUT),
    ("k_head_stride_odd", lambda a: _mut(a, k=T([16, 2, 64], strides=[136, 68, 1])), _lib.ERR_LAYOUT),
    ("negative_stride", lambda a: _mut(a, v=T([16, 2, 64], strides=[-128, 64, 1])), _lib.ERR_LAYOUT),
    ("cu_strided", lambda a: _mut(a, cu_q=T([2], I32, strides=[2])), _lib.ERR_LAYOUT),
    ("out_self_overlap", lambda a: _mut(a, out=T([16, 8, 64], strides=[0, 64, 1])), _lib.ERR_LAYOUT),
    ("out_aliases_q", lambda a: _mut(a, out=T([16, 8, 64], addr=a["q"].data)), _lib.ERR_LAYOUT),
    ("out_overlaps_k", lambda a: _mut(a, out=T([16, 8, 64], addr=a["k"].data + 1024)), _lib.ERR_LAYOUT),
]


@pytest.mark.parametrize("name,mutate,code", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_rejects(name, mutate, code):
    status = call_prefill(mutate(prefill_args()))
    assert status == code, (status, last_error())
    assert last_error(), "an error must leave a message"


def test_prefill_f32_inputs_need_f32_out():
    assert call_prefill(prefill_args(dtype=F32, out_dtype=BF16)) == _lib.ERR_DTYPE
    # bf16 inputs may write fp32 out: accepted (checked through an empty call)
    assert call_prefill(prefill_args(tq=0, out_dtype=F32)) == _lib.OK


# ----------------------------------------------------------------------------- prefill_split
def psplit_args(tq=16, hq=8, hkv=2, dim=64, b=1, splits=3, dtype=BF16):
    a = prefill_args(tq=tq, hq=hq, hkv=hkv, dim=dim, b=b, dtype=dtype)
    del a["out"]
    a.update(splits=splits, po=T([tq, hq, splits, dim], F32), pm=T([tq, hq, splits], F32),
             pd=T([tq, hq, splits], F32))
    return a


def call_psplit(a):
    return _lib.lib.sinkattn_prefill_split(R(a["q"]), R(a["k"]), R(a["v"]), R(a["sinks"]), R(a["cu_q"]),
                                           R(a["cu_k"]), a["scale"], a["causal"], a["splits"], R(a["po"]),
                                           R(a["pm"]), R(a["pd"]), None)


def test_prefill_split_empty_batch_is_ok():
    assert call_psplit(psplit_args(tq=0)) == _lib.OK
    assert call_psplit(psplit_args(tq=0, b=0)) == _lib.OK


PSPLIT_CASES = [
    ("po_null", lambda a: _mut(a, po=None), _lib.ERR_NULL),
    ("pd_null", lambda a: _mut(a, pd=None), _lib.ERR_NULL),
    ("q_null", lambda a: _mut(a, q=None), _lib.ERR_NULL),
    ("partial_bf16", lambda a: _mut(a, po=T([16, 8, 3, 64], BF16)), _lib.ERR_DTYPE),
    ("k_dtype_mismatch", lambda a: _mut(a, k=T([16, 2, 64], F32)), _lib.ERR_DTYPE),
    ("splits_zero", lambda a: _mut(a, splits=0), _lib.ERR_SHAPE),
    ("splits_negative", lambda a: _mut(a, splits=-2), _lib.ERR_SHAPE),
    ("splits_mismatch", lambda a: _mut(a, splits=4), _lib.ERR_SHAPE),
    ("po_tokens", lambda a: _mut(a, po=T([15, 8, 3, 64], F32)), _lib.ERR_SHAPE),
    ("pm_shape", lambda a: _mut(a, pm=T([16, 8, 2], F32)), _lib.ERR_SHAPE),
    ("po_rank3", lambda a: _mut(a, po=T([16, 8, 192], F32)), _lib.ERR_SHAPE),
    ("scale_nan", lambda a: _mut(a, scale=float("nan")), _lib.ERR_SHAPE),
    ("head_dim_128", lambda a: psplit_args(dim=128), _lib.ERR_UNSUPPORTED),
    ("group_3", lambda a: psplit_args(hq=6, hkv=2), _lib.ERR_UNSUPPORTED),
    ("po_strided", lambda a: _mut(a, po=T([16, 8, 3, 64], F32, strides=[4096, 256, 64, 1])), _lib.ERR_LAYOUT),
    ("pm_overlaps_pd", lambda a: _mut(a, pm=T([16, 8, 3], F32, addr=a["pd"].data + 4)), _lib.ERR_LAYOUT),
    ("po_overlaps_q", lambda a: _mut(a, po=T([16, 8, 3, 64], F32, addr=a["q"].data + 256)), _lib.ERR_LAYOUT),
    ("pd_overlaps_cu", lambda a: _mut(a, pd=T([16, 8, 3], F32, addr=a["cu_k"].data)), _lib.ERR_LAYOUT),
]


@pytest.mark.parametrize("name,mutate,code", PSPLIT_CASES, ids=[c[0] for c in PSPLIT_CASES])
def test_prefill_split_rejects(name, mutate, code):
    status = call_psplit(mutate(psplit_args()))
    assert status == code, (status, last_error())
    assert last_error()


# ----------------------------------------------------------------------------- decode_split
def split_args(b=2, hq=8, hkv=1, cap=64, chunks=4, dim=64, dtype=BF16):
    return dict(q=T([b, hq, dim], dtype), k=T([b, cap, hkv, dim], dtype), v=T([b, cap, hkv, dim], dtype),
                sinks=T([hq], F32), seqlens=T([b], I32), chunks=chunks, scale=0.125,
                po=T([b, hq, chunks, dim], F32), pm=T([b, hq, chunks], F32), pd=T([b, hq, chunks], F32))


def call_split(a):
    return _lib.lib.sinkattn_decode_split(R(a["q"]), R(a["k"]), R(a["v"]), R(a["sinks"]), R(a["seqlens"]),
                                          a["chunks"], a["scale"], R(a["po"]), R(a["pm"]), R(a["pd"]), None)


def test_split_empty_batch_is_ok():
    assert call_split(split_args(b=0)) == _lib.OK


SPLIT_CASES = [
    ("k_null", lambda a: _mut(a, k=None), _lib.ERR_NULL),
    ("seqlens_null", lambda a: _mut(a, seqlens=None), _lib.ERR_NULL),
    ("partial_bf16", lambda a: _mut(a, po=T([2, 8, 4, 64], BF16)), _lib.ERR_DTYPE),
    ("seqlens_f32", lambda a: _mut(a, seqlens=T([2], F32)), _lib.ERR_DTYPE),
    ("chunks_zero", lambda a: _mut(a, chunks=0), _lib.ERR_SHAPE),
    ("chunks_negative", lambda a: _mut(a, chunks=-3), _lib.ERR_SHAPE),
    ("partial_chunks_mismatch", lambda a: _mut(a, chunks=5), _lib.ERR_SHAPE),
    ("k_batch", lambda a: _mut(a, k=T([3, 64, 1, 64]), v=T([3, 64, 1, 64])), _lib.ERR_SHAPE),
    ("k_rank3", lambda a: _mut(a, k=T([2, 64, 64])), _lib.ERR_SHAPE),
    ("seqlens_len", lambda a: _mut(a, seqlens=T([3], I32)), _lib.ERR_SHAPE),
    ("pm_shape", lambda a: _mut(a, pm=T([2, 8, 3], F32)), _lib.ERR_SHAPE),
    ("scale_zero", lambda a: _mut(a, scale=0.0), _lib.ERR_SHAPE),
    ("group_32", lambda a: split_args(hq=32), _lib.ERR_UNSUPPORTED),
    ("group_6", lambda a: split_args(hq=6), _lib.ERR_UNSUPPORTED),
    ("head_dim_96", lambda a: split_args(dim=96), _lib.ERR_UNSUPPORTED),
    ("partial_o_strided", lambda a: _mut(a, po=T([2, 8, 4, 64], F32, strides=[4096, 512, 128, 1])), _lib.ERR_LAYOUT),
    ("k_misaligned", lambda a: _mut(a, k=T([2, 64, 1, 64], addr=(5 << 44) + 8)), _lib.ERR_LAYOUT),
    ("partial_overlaps_k", lambda a: _mut(a, po=T([2, 8, 4, 64], F32, addr=a["k"].data)), _lib.ERR_LAYOUT),
    ("pm_overlaps_pd", lambda a: _mut(a, pm=T([2, 8, 4], F32, addr=a["pd"].data + 16)), _lib.ERR_LAYOUT),
]


@pytest.mark.parametrize("name,mutate,code", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_split_rejects(name, mutate, code):
    status = call_split(mutate(split_args()))
    assert status == code, (status, last_error())
    assert last_error()


# ----------------------------------------------------------------------------- decode_merge
def merge_args(b=2, hq=8, chunks=4, dim=64, out_dtype=BF16, lse=True):
    return dict(po=T([b, hq, chunks, dim], F32), pm=T([b, hq, chunks], F32), pd=T([b, hq, chunks], F32),
                chunks=chunks, out=T([b, hq, dim], out_dtype), lse=T([b, hq], F32) if lse else None)


def call_merge(a):
    return _lib.lib.sinkattn_decode_merge(R(a["po"]), R(a["pm"]), R(a["pd"]), a["chunks"], R(a["out"]),
                                          R(a["lse"]), None)


def test_merge_empty_batch_is_ok():
    assert call_merge(merge_args(b=0)) == _lib.OK
    assert call_merge(merge_args(b=0, lse=False)) == _lib.OK


MERGE_CASES = [
    ("po_null", lambda a: _mut(a, po=None), _lib.ERR_NULL),
    ("out_null", lambda a: _mut(a, out=None), _lib.ERR_NULL),
    ("out_int", lambda a: _mut(a, out=T([2, 8, 64], I32)), _lib.ERR_DTYPE),
    ("lse_bf16", lambda a: _mut(a, lse=T([2, 8], BF16)), _lib.ERR_DTYPE),
    ("chunks_mismatch", lambda a: _mut(a, chunks=3), _lib.ERR_SHAPE),
    ("chunks_zero", lambda a: _mut(a, chunks=0), _lib.ERR_SHAPE),
    ("out_shape", lambda a: _mut(a, out=T([2, 4, 64])), _lib.ERR_SHAPE),
    ("lse_shape", lambda a: _mut(a, lse=T([2, 4], F32)), _lib.ERR_SHAPE),
    ("pd_shape", lambda a: _mut(a, pd=T([2, 8, 5], F32)), _lib.ERR_SHAPE),
    ("head_dim_32", lambda a: merge_args(dim=32), _lib.ERR_UNSUPPORTED),
    ("po_gapped", lambda a: _mut(a, po=T([2, 8, 4, 64], F32, strides=[4096, 512, 64, 1])), _lib.ERR_LAYOUT),
    ("out_overlaps_po", lambda a: _mut(a, out=T([2, 8, 64], addr=a["po"].data)), _lib.ERR_LAYOUT),
    ("lse_overlaps_out", lambda a: _mut(a, lse=T([2, 8], F32, addr=a["out"].data)), _lib.ERR_LAYOUT),
    ("pm_noncontiguous", lambda a: _mut(a, pm=T([2, 8, 4], F32, strides=[64, 8, 2])), _lib.ERR_LAYOUT),
]


@pytest.mark.parametrize("name,mutate,code", MERGE_CASES, ids=[c[0] for c in MERGE_CASES])
def test_merge_rejects(name, mutate, code):
    status = call_merge(mutate(merge_args()))
    assert status == code, (status, last_error())
    assert last_error()


def test_error_message_is_cleared_by_next_call():
    call_merge(_mut(merge_args(), chunks=0))
    assert last_error()
    assert call_merge(merge_args(b=0)) == _lib.OK
    assert last_error() == ""


# ----------------------------------------------------------------------------- fused decode
def fused_args(b=2, hq=8, hkv=1, cap=64, chunks=4, dim=64, dtype=BF16, lse=True):
    a = dict(q=T([b, hq, dim], dtype), k=T([b, cap, hkv, dim], dtype), v=T([b, cap, hkv, dim], dtype),
             sinks=T([hq], F32), seqlens=T([b], I32), chunks=chunks, scale=0.125,
             out=T([b, hq, dim], dtype), lse=T([b, hq], F32) if lse else None)
    a["ws_bytes"] = _lib.lib.sinkattn_decode_workspace_size(b, hq, hkv, chunks)
    a["ws"] = T([max(1, a["ws_bytes"] // 4)], F32).data
    return a


def call_fused(a):
    return _lib.lib.sinkattn_decode(R(a["q"]), R(a["k"]), R(a["v"]), R(a["sinks"]), R(a["seqlens"]),
                                    a["chunks"], a["scale"], a["ws"], a["ws_bytes"], R(a["out"]),
                                    R(a["lse"]), None)


def test_workspace_size_formula():
    # counters (B*Hkv u32) + partial_o + partial_m + partial_d, each rounded up to 256 bytes
    def up(x):
        return (x + 255) // 256 * 256
    for b, hq, hkv, c in [(8, 64, 8, 8), (1, 4, 1, 4), (3, 12, 3, 5), (0, 64, 8, 8)]:
        rows = b * hq * c
        want = up(b * hkv * 4) + up(rows * 64 * 4) + 2 * up(rows * 4)
        assert _lib.lib.sinkattn_decode_workspace_size(b, hq, hkv, c) == want
        assert _lib.lib.sinkattn_decode_workspace_counter_bytes(b, hkv) == up(b * hkv * 4)
    assert _lib.lib.sinkattn_decode_workspace_size(2, 8, 1, 0) == 0
    assert _lib.lib.sinkattn_decode_workspace_size(2, 8, 0, 4) == 0


def test_fused_empty_batch_is_ok():
    assert call_fused(fused_args(b=0)) == _lib.OK


FUSED_CASES = [
    ("ws_null", lambda a: _mut(a, ws=None), _lib.ERR_NULL),
    ("ws_small", lambda a: _mut(a, ws_bytes=a["ws_bytes"] - 4), _lib.ERR_SHAPE),
    ("ws_misaligned", lambda a: _mut(a, ws=a["ws"] + 64), _lib.ERR_LAYOUT),
    ("ws_overlaps_k", lambda a: _mut(a, ws=a["k"].data), _lib.ERR_LAYOUT),
    ("out_overlaps_ws", lambda a: _mut(a, out=T([2, 8, 64], addr=a["ws"] + 256)), _lib.ERR_LAYOUT),
    ("out_shape", lambda a: _mut(a, out=T([2, 4, 64])), _lib.ERR_SHAPE),
    ("out_int", lambda a: _mut(a, out=T([2, 8, 64], I32)), _lib.ERR_DTYPE),
    ("lse_shape", lambda a: _mut(a, lse=T([2, 4], F32)), _lib.ERR_SHAPE),
    ("lse_overlaps_out", lambda a: _mut(a, lse=T([2, 8], F32, addr=a["out"].data)), _lib.ERR_LAYOUT),
    ("chunks_zero", lambda a: _mut(a, chunks=0), _lib.ERR_SHAPE),
    ("group_32", lambda a: fused_args(hq=32), _lib.ERR_UNSUPPORTED),
    ("f32_in_bf16_out", lambda a: _mut(fused_args(dtype=F32), out=T([2, 8, 64], BF16)), _lib.ERR_DTYPE),
]


@pytest.mark.parametrize("name,mutate,code", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_fused_rejects(name, mutate, code):
    status = call_fused(mutate(fused_args()))
    assert status == code, (status, last_error())
    assert last_error()


# ----------------------------------------------------------------------------- decode, static workspace
def call_static(a):
    return _lib.lib.sinkattn_decode_static(R(a["q"]), R(a["k"]), R(a["v"]), R(a["sinks"]), R(a["seqlens"]),
                                           a["chunks"], a["scale"], R(a["out"]), R(a["lse"]), None)


def test_static_decode_header_limit_matches_the_workspace_formula():
    text = open(HEADER).read()
    limit = re.search(r"#define SINKATTN_DECODE_STATIC_WORKSPACE_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert limit, "SINKATTN_DECODE_STATIC_WORKSPACE_BYTES"
    assert int(limit.group(1)) << int(limit.group(2)) == 32 << 20
    # The 8 x 8192-key decode (64/8 heads, 8 chunks) and the 128-sequence mixed decode fit; a
    # problem one chunk-state row larger than the limit does not.
    assert _lib.lib.sinkattn_decode_workspace_size(8, 64, 8, 8) <= 32 << 20
    assert _lib.lib.sinkattn_decode_workspace_size(128, 64, 8, 8) <= 32 << 20


def test_static_decode_empty_batch_touches_nothing():
    # B = 0 returns before any HIP call (this container has no GPU).
    assert call_static(fused_args(b=0)) == _lib.OK


def test_static_decode_rejects_problems_beyond_its_workspace():
    # 128 sequences x 64 heads x 64 chunks of 66 floats: 138 MB of chunk states.
    a = fused_args(b=128, hq=64, hkv=8, cap=4096, chunks=64)
    assert call_static(a) == _lib.ERR_UNSUPPORTED, last_error()
    assert "static workspace" in last_error()


STATIC_CASES = [
    ("out_shape", lambda a: _mut(a, out=T([2, 4, 64])), _lib.ERR_SHAPE),
    ("out_int", lambda a: _mut(a, out=T([2, 8, 64], I32)), _lib.ERR_DTYPE),
    ("lse_overlaps_out", lambda a: _mut(a, lse=T([2, 8], F32, addr=a["out"].data)), _lib.ERR_LAYOUT),
    ("out_overlaps_k", lambda a: _mut(a, out=T([2, 8, 64], addr=a["k"].data)), _lib.ERR_LAYOUT),
    ("chunks_zero", lambda a: _mut(a, chunks=0), _lib.ERR_SHAPE),
    ("group_32", lambda a: fused_args(hq=32), _lib.ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("name,mutate,code", STATIC_CASES, ids=[c[0] for c in STATIC_CASES])
def test_static_decode_rejects(name, mutate, code):
    status = call_static(mutate(fused_args()))
    assert status == code, (status, last_error())
    assert last_error()


# ----------------------------------------------------------------------------- multi-token decode
def msplit_args(b=2, t=3, hq=8, hkv=1, cap=64, chunks=4, dim=64, dtype=BF16):
    return dict(q=T([b, t, hq, dim], dtype), k=T([b, cap, hkv, dim], dtype), v=T([b, cap, hkv, dim], dtype),
                sinks=T([hq], F32), seqlens=T([b], I32), chunks=chunks, scale=0.125,
                po=T([b * t, hq, chunks, dim], F32), pm=T([b * t, hq, chunks], F32),
                pd=T([b * t, hq, chunks], F32))


def call_msplit(a):
    return _lib.lib.sinkattn_decode_multi_split(R(a["q"]), R(a["k"]), R(a["v"]), R(a["sinks"]),
                                                R(a["seqlens"]), a["chunks"], a["scale"], R(a["po"]),
                                                R(a["pm"]), R(a["pd"]), None)


@pytest.mark.parametrize("b,t", [(0, 3), (2, 0)])
def test_multi_split_empty_is_ok(b, t):
    assert call_msplit(msplit_args(b=b, t=t)) == _lib.OK


MSPLIT_CASES = [
    ("q_rank3", lambda a: _mut(a, q=T([2, 8, 64])), _lib.ERR_SHAPE),
    ("partial_rows_b_not_bt", lambda a: _mut(a, po=T([2, 8, 4, 64], F32)), _lib.ERR_SHAPE),
    ("pm_rows_b_not_bt", lambda a: _mut(a, pm=T([2, 8, 4], F32)), _lib.ERR_SHAPE),
    ("k_batch", lambda a: _mut(a, k=T([3, 64, 1, 64]), v=T([3, 64, 1, 64])), _lib.ERR_SHAPE),
    ("sinks_len", lambda a: _mut(a, sinks=T([4], F32)), _lib.ERR_SHAPE),
    ("chunks_zero", lambda a: _mut(a, chunks=0), _lib.ERR_SHAPE),
    ("rows_over_64", lambda a: msplit_args(t=9), _lib.ERR_UNSUPPORTED),
    ("group16_t5", lambda a: msplit_args(hq=16, t=5), _lib.ERR_UNSUPPORTED),
    ("group_6", lambda a: msplit_args(hq=6), _lib.ERR_UNSUPPORTED),
    ("q_f32_k_bf16", lambda a: _mut(a, q=T([2, 3, 8, 64], F32)), _lib.ERR_DTYPE),
    ("q_token_stride_odd", lambda a: _mut(a, q=T([2, 3, 8, 64], strides=[1544, 515, 64, 1])), _lib.ERR_LAYOUT),
    ("partial_overlaps_q", lambda a: _mut(a, po=T([6, 8, 4, 64], F32, addr=a["q"].data)), _lib.ERR_LAYOUT),
]


@pytest.mark.parametrize("name,mutate,code", MSPLIT_CASES, ids=[c[0] for c in MSPLIT_CASES])
def test_multi_split_rejects(name, mutate, code):
    status = call_msplit(mutate(msplit_args()))
    assert status == code, (status, last_error())
    assert last_error()


def test_multi_split_accepts_the_largest_row_count():
    # G x T = 64 rows (8 x 8 and 16 x 4) pass validation; the B = 0 batch launches nothing.
    assert call_msplit(msplit_args(b=0, t=8, hq=8)) == _lib.OK
    assert call_msplit(msplit_args(b=0, t=4, hq=16)) == _lib.OK


def mfused_args(b=2, t=3, hq=8, hkv=1, cap=64, chunks=4, dim=64, dtype=BF16, lse=True):
    a = dict(q=T([b, t, hq, dim], dtype), k=T([b, cap, hkv, dim], dtype), v=T([b, cap, hkv, dim], dtype),
             sinks=T([hq], F32), seqlens=T([b], I32), chunks=chunks, scale=0.125,
             out=T([b, t, hq, dim], dtype), lse=T([b, t, hq], F32) if lse else None)
    a["ws_bytes"] = _lib.lib.sinkattn_decode_workspace_size(b * t, hq, hkv, chunks)
    a["ws"] = T([max(1, a["ws_bytes"] // 4)], F32).data
    return a


def call_mfused(a):
    return _lib.lib.sinkattn_decode_multi(R(a["q"]), R(a["k"]), R(a["v"]), R(a["sinks"]), R(a["seqlens"]),
                                          a["chunks"], a["scale"], a["ws"], a["ws_bytes"], R(a["out"]),
                                          R(a["lse"]), None)


def test_multi_fused_empty_is_ok():
    assert call_mfused(mfused_args(b=0)) == _lib.OK
    assert call_mfused(mfused_args(t=0)) == _lib.OK


MFUSED_CASES = [
    ("ws_sized_for_b_not_bt", lambda a: _mut(a, ws_bytes=_lib.lib.sinkattn_decode_workspace_size(2, 8, 1, 4)),
     _lib.ERR_SHAPE),
    ("out_rank3", lambda a: _mut(a, out=T([6, 8, 64])), _lib.ERR_SHAPE),
    ("out_tokens", lambda a: _mut(a, out=T([2, 2, 8, 64])), _lib.ERR_SHAPE),
    ("lse_rank2", lambda a: _mut(a, lse=T([6, 8], F32)), _lib.ERR_SHAPE),
    ("lse_tokens", lambda a: _mut(a, lse=T([2, 4, 8], F32)), _lib.ERR_SHAPE),
    ("lse_inner_stride", lambda a: _mut(a, lse=T([2, 3, 8], F32, strides=[48, 16, 2])), _lib.ERR_LAYOUT),
    ("rows_over_64", lambda a: mfused_args(t=9), _lib.ERR_UNSUPPORTED),
    ("ws_overlaps_q", lambda a: _mut(a, ws=a["q"].data), _lib.ERR_LAYOUT),
]


@pytest.mark.parametrize("name,mutate,code", MFUSED_CASES, ids=[c[0] for c in MFUSED_CASES])
def test_multi_fused_rejects(name, mutate, code):
    status = call_mfused(mutate(mfused_args()))
    assert status == code, (status, last_error())
    assert last_error()


# ----------------------------------------------------------------------------- MoE routing softmax
def moe_args(t=32, e=128, k=4, dtype=BF16, wdtype=BF16):
    return dict(logits=T([t, e], dtype), k=k, all=0, ids=T([t, k], I32), w=T([t, k], wdtype))


def call_moe(a):
    return _lib.lib.sinkattn_moe_topk_softmax(R(a["logits"]), a["k"], a["all"], R(a["ids"]), R(a["w"]), None)


def test_moe_empty_is_ok():
    assert call_moe(moe_args(t=0)) == _lib.OK


def test_moe_accepts_unaligned_rows():
    # 100 bf16 experts: 200-byte rows; element loads serve them (nothing launched for T = 0)
    assert call_moe(dict(moe_args(t=0, e=100), logits=T([0, 100], strides=[100, 1]))) == _lib.OK


MOE_CASES = [
    ("logits_null", lambda a: _mut(a, logits=None), _lib.ERR_NULL),
    ("ids_null", lambda a: _mut(a, ids=None), _lib.ERR_NULL),
    ("logits_i32", lambda a: _mut(a, logits=T([32, 128], I32)), _lib.ERR_DTYPE),
    ("ids_f32", lambda a: _mut(a, ids=T([32, 4], F32)), _lib.ERR_DTYPE),
    ("weights_i32", lambda a: _mut(a, w=T([32, 4], I32)), _lib.ERR_DTYPE),
    ("k_zero", lambda a: moe_args(k=0), _lib.ERR_SHAPE),
    ("k_over_e", lambda a: moe_args(e=3, k=4), _lib.ERR_SHAPE),
    ("ids_rows", lambda a: _mut(a, ids=T([31, 4], I32)), _lib.ERR_SHAPE),
    ("weights_cols", lambda a: _mut(a, w=T([32, 5], BF16)), _lib.ERR_SHAPE),
    ("logits_rank3", lambda a: _mut(a, logits=T([2, 16, 128])), _lib.ERR_SHAPE),
    ("e_over_256", lambda a: moe_args(e=257), _lib.ERR_UNSUPPORTED),
    ("k_over_16", lambda a: moe_args(e=64, k=17), _lib.ERR_UNSUPPORTED),
    ("logits_inner_stride", lambda a: _mut(a, logits=T([32, 128], strides=[256, 2])), _lib.ERR_LAYOUT),
    ("logits_misaligned", lambda a: _mut(a, logits=T([32, 128], addr=(7 << 44) + 1)), _lib.ERR_LAYOUT),
    ("ids_inner_stride", lambda a: _mut(a, ids=T([32, 4], I32, strides=[8, 2])), _lib.ERR_LAYOUT),
    ("weights_overlap_rows", lambda a: _mut(a, w=T([32, 4], BF16, strides=[2, 1])), _lib.ERR_LAYOUT),
    ("ids_overlap_weights", lambda a: _mut(a, ids=T([32, 4], I32, addr=a["w"].data)), _lib.ERR_LAYOUT),
    ("weights_overlap_logits", lambda a: _mut(a, w=T([32, 4], BF16, addr=a["logits"].data + 64)), _lib.ERR_LAYOUT),
]


@pytest.mark.parametrize("name,mutate,code", MOE_CASES, ids=[c[0] for c in MOE_CASES])
def test_moe_rejects(name, mutate, code):
    status = call_moe(mutate(moe_args()))
    assert status == code, (status, last_error())
    assert last_error()


# ----------------------------------------------------------------------------- linear layers
FP8 = _lib.FP8_E4M3


def lin_args(m=256, n=384, k=512, fp8=False, ydt=BF16, bias=True):
    dt = FP8 if fp8 else BF16
    a = dict(x=T([m, k], dt), w=T([n, k], dt), bias=T([n], F32) if bias else None, y=T([m, n], ydt), fp8=fp8)
    if fp8:
        a["sx"] = T([m, k // 128], F32)
        a["sw"] = T([(n + 127) // 128, k // 128], F32)
    return a


def call_lin(a):
    if a["fp8"]:
        return _lib.lib.sinkattn_linear_fp8_block_scaled(R(a["x"]), R(a["sx"]), R(a["w"]), R(a["sw"]),
                                                         R(a["bias"]), R(a["y"]), None)
    return _lib.lib.sinkattn_linear_bias(R(a["x"]), R(a["w"]), R(a["bias"]), R(a["y"]), None)


@pytest.mark.parametrize("fp8", [False, True])
def test_linear_empty_is_ok(fp8):
    assert call_lin(lin_args(m=0, fp8=fp8)) == _lib.OK
    assert call_lin(lin_args(n=0, fp8=fp8)) == _lib.OK


def test_linear_bias_may_be_null():
    assert call_lin(lin_args(m=0, bias=False)) == _lib.OK


LIN_CASES = [
    ("x_null", lambda a: _mut(a, x=None), _lib.ERR_NULL),
    ("x_f32", lambda a: _mut(a, x=T([256, 512], F32)), _lib.ERR_DTYPE),
    ("w_fp8_in_bf16_call", lambda a: _mut(a, w=T([384, 512], FP8)), _lib.ERR_DTYPE),
    ("y_i32", lambda a: _mut(a, y=T([256, 384], I32)), _lib.ERR_DTYPE),
    ("bias_bf16", lambda a: _mut(a, bias=T([384], BF16)), _lib.ERR_DTYPE),
    ("k_mismatch", lambda a: _mut(a, w=T([384, 448])), _lib.ERR_SHAPE),
    ("k_not_multiple_of_64", lambda a: lin_args(k=96), _lib.ERR_SHAPE),
    ("y_shape", lambda a: _mut(a, y=T([256, 383])), _lib.ERR_SHAPE),
    ("bias_len", lambda a: _mut(a, bias=T([383], F32)), _lib.ERR_SHAPE),
    ("x_rank3", lambda a: _mut(a, x=T([2, 128, 512])), _lib.ERR_SHAPE),
    ("x_row_unaligned", lambda a: _mut(a, x=T([256, 512], strides=[516, 1])), _lib.ERR_LAYOUT),
    ("x_rows_overlap", lambda a: _mut(a, x=T([256, 512], strides=[8, 1])), _lib.ERR_LAYOUT),
    ("y_inner_stride", lambda a: _mut(a, y=T([256, 384], strides=[768, 2])), _lib.ERR_LAYOUT),
    ("y_overlaps_x", lambda a: _mut(a, y=T([256, 384], addr=a["x"].data)), _lib.ERR_LAYOUT),
    ("fp8_k_not_multiple_of_128", lambda a: lin_args(k=192, fp8=True), _lib.ERR_SHAPE),
    ("fp8_scale_x_shape", lambda a: _mut(lin_args(fp8=True), sx=T([256, 3], F32)), _lib.ERR_SHAPE),
    ("fp8_scale_w_shape", lambda a: _mut(lin_args(fp8=True), sw=T([2, 4], F32)), _lib.ERR_SHAPE),
    ("fp8_scale_bf16", lambda a: _mut(lin_args(fp8=True), sx=T([256, 4], BF16)), _lib.ERR_DTYPE),
    ("fp8_bf16_operand", lambda a: _mut(lin_args(fp8=True), x=T([256, 512], BF16)), _lib.ERR_DTYPE),
    ("fp8_scale_null", lambda a: _mut(lin_args(fp8=True), sw=None), _lib.ERR_NULL),
]


@pytest.mark.parametrize("name,mutate,code", LIN_CASES, ids=[c[0] for c in LIN_CASES])
def test_linear_rejects(name, mutate, code):
    status = call_lin(mutate(lin_args()))
    assert status == code, (status, last_error())
    assert last_error()
