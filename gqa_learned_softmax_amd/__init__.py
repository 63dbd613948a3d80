"""Sink attention for AMD MI355X: Python face of the libsinkattn C ABI (include/sinkattn.h).

Grouped-query attention whose softmax carries one learned logit per query head (the "sink") that
adds to the denominator and has no value vector, as described in the blog post "GPT-OSS on Day 0"
(Perplexity), section "Kernels for GPT-OSS", subsection "Sink attention".

Each function marshals torch tensors into descriptors and calls the library on the current HIP
stream. Allocation of outputs (when not given) is the only other thing done here.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import SinkAttnError  # noqa: F401

__all__ = ["prefill", "prefill_split", "prefill_kv_split", "decode_split", "decode_merge", "decode",
           "decode_fused", "decode_workspace", "decode_static", "decode_multi_split", "decode_multi", "decode_multi_fused",
           "moe_topk_softmax", "linear_bias", "linear_fp8_block_scaled", "plan_decode", "plan_prefill",
           "SinkAttnError", "version"]


def version() -> int:
    return _lib.lib.sinkattn_version()


def prefill(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, scale, causal=True, out=None,
            out_dtype=None):
    """``sinkattn_prefill``: q [Tq, Hq, D], k/v [Tk, Hkv, D], sinks [Hq] f32, cu_seqlens [B+1] i32."""
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    dev = _lib.require_device(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, out)
    d = [_lib.describe(t) for t in (q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, out)]
    _lib.check(_lib.lib.sinkattn_prefill(
        _lib.ref(d[0]), _lib.ref(d[1]), _lib.ref(d[2]), _lib.ref(d[3]), _lib.ref(d[4]),
        _lib.ref(d[5]), float(scale), 1 if causal else 0, _lib.ref(d[6]), _lib.stream_handle(dev)))
    return out


def prefill_split(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, scale, causal, num_splits,
                  partial_o=None, partial_m=None, partial_d=None):
    """``sinkattn_prefill_split``: returns (partial_o [Tq,Hq,S,D], partial_m [Tq,Hq,S], partial_d)."""
    tq, hq, dim = q.shape
    if partial_o is None:
        partial_o = torch.empty((tq, hq, num_splits, dim), dtype=torch.float32, device=q.device)
    if partial_m is None:
        partial_m = torch.empty((tq, hq, num_splits), dtype=torch.float32, device=q.device)
    if partial_d is None:
        partial_d = torch.empty((tq, hq, num_splits), dtype=torch.float32, device=q.device)
    dev = _lib.require_device(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, partial_o, partial_m, partial_d)
    d = [_lib.describe(t) for t in (q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, partial_o, partial_m, partial_d)]
    _lib.check(_lib.lib.sinkattn_prefill_split(
        _lib.ref(d[0]), _lib.ref(d[1]), _lib.ref(d[2]), _lib.ref(d[3]), _lib.ref(d[4]), _lib.ref(d[5]),
        float(scale), 1 if causal else 0, int(num_splits), _lib.ref(d[6]), _lib.ref(d[7]), _lib.ref(d[8]),
        _lib.stream_handle(dev)))
    return partial_o, partial_m, partial_d


def prefill_kv_split(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, scale, causal, num_splits, out=None,
                     return_lse=False):
    """Split-KV prefill then the log-sum-exp merge (partials allocated with torch); out [Tq, Hq, D]."""
    po, pm, pd = prefill_split(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, scale, causal, num_splits)
    return decode_merge(po, pm, pd, out=out, out_dtype=q.dtype, return_lse=return_lse)


def decode_split(q, k, v, sinks, seqlens_k, num_chunks, scale, partial_o=None, partial_m=None,
                 partial_d=None):
    """``sinkattn_decode_split``: returns (partial_o [B,Hq,C,D], partial_m [B,Hq,C], partial_d)."""
    batch, hq, dim = q.shape
    if partial_o is None:
        partial_o = torch.empty((batch, hq, num_chunks, dim), dtype=torch.float32, device=q.device)
    if partial_m is None:
        partial_m = torch.empty((batch, hq, num_chunks), dtype=torch.float32, device=q.device)
    if partial_d is None:
        partial_d = torch.empty((batch, hq, num_chunks), dtype=torch.float32, device=q.device)
    dev = _lib.require_device(q, k, v, sinks, seqlens_k, partial_o, partial_m, partial_d)
    d = [_lib.describe(t) for t in (q, k, v, sinks, seqlens_k, partial_o, partial_m, partial_d)]
    _lib.check(_lib.lib.sinkattn_decode_split(
        _lib.ref(d[0]), _lib.ref(d[1]), _lib.ref(d[2]), _lib.ref(d[3]), _lib.ref(d[4]),
        int(num_chunks), float(scale), _lib.ref(d[5]), _lib.ref(d[6]), _lib.ref(d[7]),
        _lib.stream_handle(dev)))
    return partial_o, partial_m, partial_d


def decode_merge(partial_o, partial_m, partial_d, out=None, lse=None, out_dtype=torch.bfloat16,
                 return_lse=False):
    """``sinkattn_decode_merge``: out [B, Hq, D] (and lse [B, Hq] f32 when requested)."""
    batch, hq, chunks, dim = partial_o.shape
    if out is None:
        out = torch.empty((batch, hq, dim), dtype=out_dtype, device=partial_o.device)
    if lse is None and return_lse:
        lse = torch.empty((batch, hq), dtype=torch.float32, device=partial_o.device)
    dev = _lib.require_device(partial_o, partial_m, partial_d, out, lse)
    d = [_lib.describe(t) for t in (partial_o, partial_m, partial_d, out, lse)]
    _lib.check(_lib.lib.sinkattn_decode_merge(
        _lib.ref(d[0]), _lib.ref(d[1]), _lib.ref(d[2]), int(chunks), _lib.ref(d[3]),
        _lib.ref(d[4]), _lib.stream_handle(dev)))
    return (out, lse) if (return_lse or lse is not None) else out


def decode(q, k, v, sinks, seqlens_k, num_chunks, scale, out=None, return_lse=False):
    """Split then merge on the current stream (partials allocated with torch)."""
    po, pm, pd = decode_split(q, k, v, sinks, seqlens_k, num_chunks, scale)
    return decode_merge(po, pm, pd, out=out, out_dtype=q.dtype, return_lse=return_lse)


def decode_workspace(batch, num_q_heads, num_kv_heads, num_chunks, device):
    """A zeroed workspace for ``decode_fused`` (reusable across calls on one stream)."""
    size = _lib.lib.sinkattn_decode_workspace_size(batch, num_q_heads, num_kv_heads, num_chunks)
    return torch.zeros(max(int(size), 1), dtype=torch.uint8, device=device)


def decode_fused(q, k, v, sinks, seqlens_k, num_chunks, scale, workspace, out=None, lse=None,
                 return_lse=False):
    """``sinkattn_decode``: split-KV decode and merge through ``workspace`` (one launch when the split
    grid has at most one work-group per compute unit); out [B, Hq, D]."""
    batch, hq, dim = q.shape
    if out is None:
        out = torch.empty((batch, hq, dim), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((batch, hq), dtype=torch.float32, device=q.device)
    dev = _lib.require_device(q, k, v, sinks, seqlens_k, workspace, out, lse)
    d = [_lib.describe(t) for t in (q, k, v, sinks, seqlens_k, out, lse)]
    _lib.check(_lib.lib.sinkattn_decode(
        _lib.ref(d[0]), _lib.ref(d[1]), _lib.ref(d[2]), _lib.ref(d[3]), _lib.ref(d[4]),
        int(num_chunks), float(scale), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _lib.ref(d[5]), _lib.ref(d[6]), _lib.stream_handle(dev)))
    return (out, lse) if (return_lse or lse is not None) else out


def decode_static(q, k, v, sinks, seqlens_k, num_chunks, scale, out=None, lse=None, return_lse=False):
    """``sinkattn_decode_static``: as ``decode_fused`` with the library's own device workspace
    (nothing allocated by the library; ``out``/``lse`` are allocated here when not given)."""
    batch, hq, dim = q.shape
    if out is None:
        out = torch.empty((batch, hq, dim), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((batch, hq), dtype=torch.float32, device=q.device)
    dev = _lib.require_device(q, k, v, sinks, seqlens_k, out, lse)
    d = [_lib.describe(t) for t in (q, k, v, sinks, seqlens_k, out, lse)]
    _lib.check(_lib.lib.sinkattn_decode_static(
        _lib.ref(d[0]), _lib.ref(d[1]), _lib.ref(d[2]), _lib.ref(d[3]), _lib.ref(d[4]),
        int(num_chunks), float(scale), _lib.ref(d[5]), _lib.ref(d[6]), _lib.stream_handle(dev)))
    return (out, lse) if (return_lse or lse is not None) else out


def decode_multi_split(q, k, v, sinks, seqlens_k, num_chunks, scale, partial_o=None, partial_m=None,
                       partial_d=None):
    """``sinkattn_decode_multi_split``: q [B, T, Hq, D]; returns (partial_o [B*T, Hq, C, D],
    partial_m [B*T, Hq, C], partial_d [B*T, Hq, C])."""
    batch, q_len, hq, dim = q.shape
    rows = batch * q_len
    if partial_o is None:
        partial_o = torch.empty((rows, hq, num_chunks, dim), dtype=torch.float32, device=q.device)
    if partial_m is None:
        partial_m = torch.empty((rows, hq, num_chunks), dtype=torch.float32, device=q.device)
    if partial_d is None:
        partial_d = torch.empty((rows, hq, num_chunks), dtype=torch.float32, device=q.device)
    dev = _lib.require_device(q, k, v, sinks, seqlens_k, partial_o, partial_m, partial_d)
    d = [_lib.describe(t) for t in (q, k, v, sinks, seqlens_k, partial_o, partial_m, partial_d)]
    _lib.check(_lib.lib.sinkattn_decode_multi_split(
        _lib.ref(d[0]), _lib.ref(d[1]), _lib.ref(d[2]), _lib.ref(d[3]), _lib.ref(d[4]),
        int(num_chunks), float(scale), _lib.ref(d[5]), _lib.ref(d[6]), _lib.ref(d[7]),
        _lib.stream_handle(dev)))
    return partial_o, partial_m, partial_d


def decode_multi(q, k, v, sinks, seqlens_k, num_chunks, scale, return_lse=False):
    """Multi-token split then merge (partials allocated with torch); out [B, T, Hq, D]."""
    batch, q_len, hq, dim = q.shape
    po, pm, pd = decode_multi_split(q, k, v, sinks, seqlens_k, num_chunks, scale)
    res = decode_merge(po, pm, pd, out_dtype=q.dtype, return_lse=return_lse)
    if return_lse:
        out, lse = res
        return out.view(batch, q_len, hq, dim), lse.view(batch, q_len, hq)
    return res.view(batch, q_len, hq, dim)


def decode_multi_fused(q, k, v, sinks, seqlens_k, num_chunks, scale, workspace, out=None, lse=None,
                       return_lse=False):
    """``sinkattn_decode_multi``: out [B, T, Hq, D]; ``workspace`` from
    ``decode_workspace(B * T, Hq, Hkv, num_chunks, device)``."""
    batch, q_len, hq, dim = q.shape
    if out is None:
        out = torch.empty((batch, q_len, hq, dim), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((batch, q_len, hq), dtype=torch.float32, device=q.device)
    dev = _lib.require_device(q, k, v, sinks, seqlens_k, workspace, out, lse)
    d = [_lib.describe(t) for t in (q, k, v, sinks, seqlens_k, out, lse)]
    _lib.check(_lib.lib.sinkattn_decode_multi(
        _lib.ref(d[0]), _lib.ref(d[1]), _lib.ref(d[2]), _lib.ref(d[3]), _lib.ref(d[4]),
        int(num_chunks), float(scale), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _lib.ref(d[5]), _lib.ref(d[6]), _lib.stream_handle(dev)))
    return (out, lse) if (return_lse or lse is not None) else out


def _launches(buf, count):
    return [{"kernel": buf[i].kernel.decode(), "grid": int(buf[i].grid), "block": int(buf[i].block)}
            for i in range(count.value)]


def plan_decode(q, k, v, sinks, seqlens_k, num_chunks, scale, form="split"):
    """``sinkattn_plan_decode``: the launches of ``decode_split`` / ``decode_multi_split``
    (``form="split"``) or of ``decode_fused`` / ``decode_multi_fused`` / ``decode_static``
    (``form="decode"``) for these inputs, as ``[{"kernel", "grid", "block"}, ...]``. Nothing is
    launched and no tensor is read, so CPU tensors of the right shapes and strides will do."""
    forms = {"split": _lib.PLAN_DECODE_SPLIT, "decode": _lib.PLAN_DECODE}
    buf = (_lib.Launch * 2)()
    count = ctypes.c_int(0)
    d = [_lib.describe(t) for t in (q, k, v, sinks, seqlens_k)]
    _lib.check(_lib.lib.sinkattn_plan_decode(
        _lib.ref(d[0]), _lib.ref(d[1]), _lib.ref(d[2]), _lib.ref(d[3]), _lib.ref(d[4]),
        int(num_chunks), float(scale), forms[form], buf, ctypes.byref(count)))
    return _launches(buf, count)


def plan_prefill(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, scale, causal=True, num_splits=0):
    """``sinkattn_plan_prefill``: the launch of ``prefill`` (``num_splits=0``) or of
    ``prefill_split`` for these inputs (CPU tensors will do, as for ``plan_decode``)."""
    buf = (_lib.Launch * 1)()
    count = ctypes.c_int(0)
    d = [_lib.describe(t) for t in (q, k, v, sinks, cu_seqlens_q, cu_seqlens_k)]
    _lib.check(_lib.lib.sinkattn_plan_prefill(
        _lib.ref(d[0]), _lib.ref(d[1]), _lib.ref(d[2]), _lib.ref(d[3]), _lib.ref(d[4]), _lib.ref(d[5]),
        float(scale), 1 if causal else 0, int(num_splits), buf, ctypes.byref(count)))
    return _launches(buf, count)


def moe_topk_softmax(logits, top_k, over_all_experts=False, ids=None, weights=None,
                     weights_dtype=torch.bfloat16):
    """``sinkattn_moe_topk_softmax``: logits [T, E]; returns (ids [T, K] int32, weights [T, K])."""
    tokens = logits.shape[0]
    if ids is None:
        ids = torch.empty((tokens, top_k), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((tokens, top_k), dtype=weights_dtype, device=logits.device)
    dev = _lib.require_device(logits, ids, weights)
    d = [_lib.describe(t) for t in (logits, ids, weights)]
    _lib.check(_lib.lib.sinkattn_moe_topk_softmax(
        _lib.ref(d[0]), int(top_k), 1 if over_all_experts else 0, _lib.ref(d[1]), _lib.ref(d[2]),
        _lib.stream_handle(dev)))
    return ids, weights


def linear_bias(x, w, bias=None, out=None, out_dtype=torch.bfloat16):
    """``sinkattn_linear_bias``: y [M, N] = x [M, K] w[N, K]^T + bias [N] (bf16 operands)."""
    if out is None:
        out = torch.empty((x.shape[0], w.shape[0]), dtype=out_dtype, device=x.device)
    dev = _lib.require_device(x, w, bias, out)
    d = [_lib.describe(t) for t in (x, w, bias, out)]
    _lib.check(_lib.lib.sinkattn_linear_bias(_lib.ref(d[0]), _lib.ref(d[1]), _lib.ref(d[2]), _lib.ref(d[3]),
                                             _lib.stream_handle(dev)))
    return out


def linear_fp8_block_scaled(x, scale_x, w, scale_w, bias=None, out=None, out_dtype=torch.bfloat16):
    """``sinkattn_linear_fp8_block_scaled``: x [M, K], w [N, K] float8_e4m3fn; scale_x [M, K/128],
    scale_w [ceil(N/128), K/128] fp32; y [M, N]."""
    if out is None:
        out = torch.empty((x.shape[0], w.shape[0]), dtype=out_dtype, device=x.device)
    dev = _lib.require_device(x, scale_x, w, scale_w, bias, out)
    d = [_lib.describe(t) for t in (x, scale_x, w, scale_w, bias, out)]
    _lib.check(_lib.lib.sinkattn_linear_fp8_block_scaled(
        _lib.ref(d[0]), _lib.ref(d[1]), _lib.ref(d[2]), _lib.ref(d[3]), _lib.ref(d[4]), _lib.ref(d[5]),
        _lib.stream_handle(dev)))
    return out
