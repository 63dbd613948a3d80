"""Accepted calls through the C ABI, checked on the host: what each call hands its kernel launcher.

Runs only against the host-only build of the ABI layer (api.cpp linked with stub launchers that
record each launch instead of launching; SINKATTN_LIBRARY names it), which the test module
tests/test_host_abi.py builds with AddressSanitizer and UndefinedBehaviorSanitizer and runs this
file under. Descriptors carry placeholder addresses that nothing dereferences.

Checked: the decode grid (KV heads per work-group, key split, work-groups), the chunk size, the
single-launch decision of sinkattn_decode and the carving of its workspace, the static workspace
of sinkattn_decode_static, the prefill grid bound, the merge variant, the plan queries against the
launches actually made, and the launch-failure path.
"""
from __future__ import annotations

import ctypes
import json
import math

import numpy as np
import pytest

from gqa_learned_softmax_amd import _lib
from gqa_learned_softmax_amd._lib import BF16, F32, I32, Tensor

if not hasattr(_lib.lib, "sinkattn_stub_take_log"):
    pytest.skip("needs the host-only build of the ABI layer (SINKATTN_LIBRARY)", allow_module_level=True)

_lib.lib.sinkattn_stub_take_log.argtypes = [ctypes.c_char_p, ctypes.c_size_t]
_lib.lib.sinkattn_stub_take_log.restype = ctypes.c_size_t
_lib.lib.sinkattn_stub_fail_next.argtypes = [ctypes.c_int]
_lib.lib.sinkattn_stub_fail_next.restype = None

COMPUTE_UNITS = 256
HIP_ERROR_INVALID_CONFIGURATION = 9

_next = [1 << 40]


def T(shape, dtype=BF16, strides=None):
    d = Tensor()
    d.data = _next[0]
    _next[0] += 1 << 36  # 64 GiB apart: no two descriptors overlap
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


def take_log():
    n = _lib.lib.sinkattn_stub_take_log(None, 0)
    assert n == 0, "records left over from an earlier call"
    return []


def records():
    buf = ctypes.create_string_buffer(1 << 20)
    n = _lib.lib.sinkattn_stub_take_log(buf, len(buf))
    assert n < len(buf)
    return [json.loads(line) for line in buf.value.decode().splitlines()]


def ok(status):
    assert status == _lib.OK, (status, _lib.lib.sinkattn_last_error().decode())


# ----------------------------------------------------------------------------- decode
def decode_inputs(b, hq, hkv, cap, q_len=1, dtype=BF16, head_major=False):
    q = T([b, hq, 64] if q_len == 1 else [b, q_len, hq, 64], dtype)
    if head_major:  # cache laid out [B, Hkv, cap, D], viewed as [B, cap, Hkv, D]
        strides = [hkv * cap * 64, 64, cap * 64, 1]
        k, v = T([b, cap, hkv, 64], dtype, strides), T([b, cap, hkv, 64], dtype, strides)
    else:
        k, v = T([b, cap, hkv, 64], dtype), T([b, cap, hkv, 64], dtype)
    return q, k, v, T([hq], F32), T([b], I32)


def split_call(b, hq, hkv, cap, chunks, q_len=1, dtype=BF16, head_major=False):
    q, k, v, s, sl = decode_inputs(b, hq, hkv, cap, q_len, dtype, head_major)
    rows = b * q_len
    po, pm, pd = T([rows, hq, chunks, 64], F32), T([rows, hq, chunks], F32), T([rows, hq, chunks], F32)
    take_log()
    fn = _lib.lib.sinkattn_decode_split if q_len == 1 else _lib.lib.sinkattn_decode_multi_split
    ok(fn(R(q), R(k), R(v), R(s), R(sl), chunks, 0.125, R(po), R(pm), R(pd), None))
    return records(), (q, k, v, s, sl), (po, pm, pd)


def expected_shape(b, hq, hkv, chunks, q_len, adjacent):
    """The grid rule, stated once more from its description: four KV heads per work-group when the
    cache rows hold them adjacently and that still leaves two work-groups per compute unit, two
    when every compute unit still gets one, else one; key split when G x T <= 16."""
    quad, paired = b * (hkv // 4) * chunks, b * (hkv // 2) * chunks
    if hkv % 4 == 0 and adjacent and quad >= 2 * COMPUTE_UNITS:
        heads, groups = 4, quad
    elif hkv % 2 == 0 and adjacent and paired >= COMPUTE_UNITS:
        heads, groups = 2, paired
    else:
        heads, groups = 1, b * hkv * chunks
    return heads, (hq // hkv) * q_len <= 16, groups


def expected_private(heads, key_split, groups):
    """Private per-wave staging: pairs of KV heads, key split, a single round of work-groups."""
    return heads == 2 and key_split and groups <= COMPUTE_UNITS


SPLIT_CASES = [
    # name, B, Hq, Hkv, capacity, chunks, T, head-major cache
    ("decode_8x8192", 8, 64, 8, 8192, 8, 1, False),
    ("long_decode_32x32768", 32, 64, 8, 32768, 16, 1, False),
    ("mixed_decode_128x8192", 128, 64, 8, 8192, 8, 1, False),
    ("one_sequence", 1, 64, 8, 4096, 4, 1, False),
    ("paired_just_fits", 4, 64, 8, 8192, 16, 1, False),
    ("quad_just_fits", 16, 64, 8, 8192, 16, 1, False),
    ("head_major", 32, 64, 8, 8192, 16, 1, True),
    ("odd_kv_heads", 64, 12, 3, 2048, 8, 1, False),
    ("group_16", 8, 128, 8, 1024, 5, 1, False),
    ("group_1", 8, 8, 8, 1000, 3, 1, False),
    ("multi_t2_g8", 8, 64, 8, 8192, 8, 2, False),
    ("multi_t4_g16", 2, 64, 4, 8192, 8, 4, False),
    ("capacity_not_multiple", 3, 64, 8, 1001, 7, 1, False),
]


@pytest.mark.parametrize("name,b,hq,hkv,cap,chunks,t,hm", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_decode_split_launch(name, b, hq, hkv, cap, chunks, t, hm):
    recs, (q, k, v, s, sl), (po, pm, pd) = split_call(b, hq, hkv, cap, chunks, t, head_major=hm)
    assert len(recs) == 1
    r = recs[0]
    heads, key_split, groups = expected_shape(b, hq, hkv, chunks, t, adjacent=not hm)
    assert r["launcher"] == "decode_split_bf16"
    assert (r["heads_per_group"], r["key_split"], r["grid"]) == (heads, key_split, groups)
    assert r["block"] == 256 * heads
    priv = expected_private(heads, key_split, groups)
    assert r["private_staging"] == priv
    assert r["kernel"] == (f"decode_split_bf16_kernel<{heads}, false, {str(key_split).lower()}, "
                           f"{str(priv).lower()}>")
    assert r["chunk_size"] == math.ceil(cap / chunks) and r["capacity"] == cap
    assert (r["batch"], r["q_len"], r["num_chunks"]) == (b, t, chunks)
    assert (r["partial_o"], r["partial_m"], r["partial_d"]) == (po.data, pm.data, pd.data)
    # Every key of every sequence falls in exactly one chunk.
    assert r["chunk_size"] * chunks >= cap and r["chunk_size"] * (chunks - 1) < cap


def test_decode_split_grid_of_the_known_workloads():
    expect = {"decode_8x8192": ("decode_split_bf16_kernel<2, false, true, true>", 256, 512),
              "long_decode_32x32768": ("decode_split_bf16_kernel<4, false, true, false>", 1024, 1024),
              "mixed_decode_128x8192": ("decode_split_bf16_kernel<4, false, true, false>", 2048, 1024)}
    for name, b, hq, hkv, cap, chunks, t, hm in SPLIT_CASES:
        if name in expect:
            recs, _, _ = split_call(b, hq, hkv, cap, chunks, t, head_major=hm)
            assert (recs[0]["kernel"], recs[0]["grid"], recs[0]["block"]) == expect[name], name


def workspace_offsets(rows, hq, hkv_rows, chunks):
    def a256(x):
        return (x + 255) // 256 * 256
    counters = 0
    po = a256(hkv_rows * 4)
    pm = po + a256(rows * hq * chunks * 64 * 4)
    pd = pm + a256(rows * hq * chunks * 4)
    total = pd + a256(rows * hq * chunks * 4)
    return counters, po, pm, pd, total


FUSED_CASES = [
    # name, B, Hq, Hkv, capacity, chunks, T, dtype
    ("one_round_8x8192", 8, 64, 8, 8192, 8, 1, BF16),
    ("two_rounds_16x8192", 16, 64, 8, 8192, 8, 1, BF16),
    ("long_32x32768", 32, 64, 8, 32768, 16, 1, BF16),
    ("fp32_reference", 2, 8, 2, 256, 4, 1, F32),
    ("multi_t4", 8, 64, 8, 8192, 8, 4, BF16),
    ("multi_t8_large", 16, 64, 8, 8192, 8, 8, BF16),
]


@pytest.mark.parametrize("name,b,hq,hkv,cap,chunks,t,dt", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_decode_single_launch_decision_and_workspace(name, b, hq, hkv, cap, chunks, t, dt):
    q, k, v, s, sl = decode_inputs(b, hq, hkv, cap, t, dt)
    out_shape = [b, hq, 64] if t == 1 else [b, t, hq, 64]
    out, lse = T(out_shape, dt), T(out_shape[:-1], F32)
    counters, po, pm, pd, total = workspace_offsets(b * t, hq, b * t * hkv, chunks)
    assert _lib.lib.sinkattn_decode_workspace_size(b * t, hq, hkv, chunks) == total
    ws = 1 << 47
    take_log()
    fn = _lib.lib.sinkattn_decode if t == 1 else _lib.lib.sinkattn_decode_multi
    ok(fn(R(q), R(k), R(v), R(s), R(sl), chunks, 0.125, ws, total, R(out), R(lse), None))
    recs = records()
    heads, key_split, groups = expected_shape(b, hq, hkv, chunks, t, adjacent=True)
    one_round = dt == BF16 and groups <= COMPUTE_UNITS
    if one_round:
        assert [r["launcher"] for r in recs] == ["decode_fused_bf16"]
        priv = str(expected_private(heads, key_split, groups)).lower()
        assert recs[0]["kernel"] == f"decode_split_bf16_kernel<{heads}, true, {str(key_split).lower()}, {priv}>"
        assert recs[0]["counters"] == ws + counters
        assert (recs[0]["out"], recs[0]["lse"]) == (out.data, lse.data)
    else:
        split = "decode_split_bf16" if dt == BF16 else "decode_split_f32"
        assert [r["launcher"] for r in recs] == [split, "decode_merge"]
        merge = recs[1]
        assert (merge["batch"], merge["q_len"], merge["num_chunks"]) == (b * t, t, chunks)
        assert (merge["out"], merge["lse"]) == (out.data, lse.data)
        assert (merge["partial_o"], merge["partial_m"], merge["partial_d"]) == (ws + po, ws + pm, ws + pd)
    first = recs[0]
    assert (first["partial_o"], first["partial_m"], first["partial_d"]) == (ws + po, ws + pm, ws + pd)
    assert first["chunk_size"] == math.ceil(cap / chunks)


def test_static_decode_runs_on_the_library_workspace():
    b, hq, hkv, cap, chunks = 8, 64, 8, 8192, 8
    q, k, v, s, sl = decode_inputs(b, hq, hkv, cap)
    out, lse = T([b, hq, 64]), T([b, hq], F32)
    take_log()
    ok(_lib.lib.sinkattn_decode_static(R(q), R(k), R(v), R(s), R(sl), chunks, 0.125, R(out), R(lse), None))
    recs = records()
    assert [r["launcher"] for r in recs] == ["static_workspace", "decode_fused_bf16"]
    base = recs[0]["address"]
    _, po, pm, pd, _ = workspace_offsets(b, hq, b * hkv, chunks)
    assert recs[1]["counters"] == base
    assert (recs[1]["partial_o"], recs[1]["partial_m"], recs[1]["partial_d"]) == (base + po, base + pm, base + pd)


# ----------------------------------------------------------------------------- merge
MERGE_CASES = [(8, 64, 8), (128, 64, 8), (127, 64, 8), (128, 64, 17), (512, 64, 16), (3, 4, 1)]


@pytest.mark.parametrize("b,hq,chunks", MERGE_CASES)
def test_merge_variant_and_grid(b, hq, chunks):
    po, pm, pd = T([b, hq, chunks, 64], F32), T([b, hq, chunks], F32), T([b, hq, chunks], F32)
    out = T([b, hq, 64])
    take_log()
    ok(_lib.lib.sinkattn_decode_merge(R(po), R(pm), R(pd), chunks, R(out), None, None))
    (r,) = records()
    rows = b * hq
    if rows >= 8192 and chunks <= 16:
        assert (r["kernel"], r["grid"]) == ("decode_merge_x4_kernel", math.ceil(rows / 16))
    else:
        assert (r["kernel"], r["grid"]) == ("decode_merge_kernel", math.ceil(rows / 4))
    assert r["block"] == 256


# ----------------------------------------------------------------------------- prefill
def prefill_inputs(lens_q, lens_k, hq, hkv, dtype=BF16):
    tq, tk = int(sum(lens_q)), int(sum(lens_k))
    q, k, v = T([tq, hq, 64], dtype), T([tk, hkv, 64], dtype), T([tk, hkv, 64], dtype)
    return q, k, v, T([hq], F32), T([len(lens_q) + 1], I32), T([len(lens_k) + 1], I32)


@pytest.mark.parametrize("group", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_prefill_grid_bounds_every_tile(group, seed):
    """The grid is taken without reading cu_seqlens; it must cover every sequence's query tiles."""
    rng = np.random.default_rng(seed * 31 + group)
    n = int(rng.integers(1, 40))
    lens = rng.integers(0, 3000, n)
    lens[rng.integers(0, n)] = int(rng.integers(1, 300))  # a short one
    hkv = 8 if group <= 8 else 4
    hq = hkv * group
    ins = prefill_inputs(lens, lens, hq, hkv)
    out = T([int(lens.sum()), hq, 64])
    take_log()
    ok(_lib.lib.sinkattn_prefill(*[R(d) for d in ins], 0.125, 1, R(out), None))
    recs = records()
    if lens.sum() == 0:
        assert recs == []
        return
    (r,) = recs
    ppt = 256 // group
    assert r["positions_per_tile"] == ppt and r["block"] == 256 and r["kernel"] == "prefill_bf16_kernel<false>"
    needed = int(sum(math.ceil(int(x) / ppt) for x in lens))
    assert r["tiles"] >= needed
    assert r["grid"] == r["tiles"] * hkv
    assert r["tiles"] == math.ceil(int(lens.sum()) / ppt) + n


def test_prefill_split_grid_and_plan():
    lens_q, lens_k = [512, 7, 300], [32768, 4000, 300]
    ins = prefill_inputs(lens_q, lens_k, 64, 8)
    tq = sum(lens_q)
    for splits in (1, 4, 9):
        po, pm, pd = T([tq, 64, splits, 64], F32), T([tq, 64, splits], F32), T([tq, 64, splits], F32)
        take_log()
        ok(_lib.lib.sinkattn_prefill_split(*[R(d) for d in ins], 0.125, 1, splits, R(po), R(pm), R(pd), None))
        (r,) = records()
        assert r["kernel"] == "prefill_bf16_kernel<true>" and r["num_splits"] == splits
        assert r["grid"] == (math.ceil(tq / 32) + 3) * 8 * splits
        buf, count = (_lib.Launch * 1)(), ctypes.c_int(0)
        ok(_lib.lib.sinkattn_plan_prefill(*[R(d) for d in ins], 0.125, 1, splits, buf, ctypes.byref(count)))
        assert count.value == 1
        assert (buf[0].kernel.decode(), buf[0].grid, buf[0].block) == (r["kernel"], r["grid"], r["block"])


# ----------------------------------------------------------------------------- plan queries
@pytest.mark.parametrize("name,b,hq,hkv,cap,chunks,t,dt", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_decode_plan_matches_the_launches(name, b, hq, hkv, cap, chunks, t, dt):
    q, k, v, s, sl = decode_inputs(b, hq, hkv, cap, t, dt)
    out_shape = [b, hq, 64] if t == 1 else [b, t, hq, 64]
    out = T(out_shape, dt)
    total = _lib.lib.sinkattn_decode_workspace_size(b * t, hq, hkv, chunks)
    take_log()
    fn = _lib.lib.sinkattn_decode if t == 1 else _lib.lib.sinkattn_decode_multi
    ok(fn(R(q), R(k), R(v), R(s), R(sl), chunks, 0.125, 1 << 47, total, R(out), None, None))
    launched = [(r["kernel"], r["grid"], r["block"]) for r in records()]
    buf, count = (_lib.Launch * 2)(), ctypes.c_int(0)
    ok(_lib.lib.sinkattn_plan_decode(R(q), R(k), R(v), R(s), R(sl), chunks, 0.125, _lib.PLAN_DECODE, buf,
                                     ctypes.byref(count)))
    assert [(buf[i].kernel.decode(), buf[i].grid, buf[i].block) for i in range(count.value)] == launched
    assert records() == []  # the plan query launched nothing


def test_plan_rejects_what_the_call_rejects():
    q, k, v, s, sl = decode_inputs(8, 64, 8, 8192)
    bad_sinks = T([63], F32)
    buf, count = (_lib.Launch * 2)(), ctypes.c_int(7)
    st = _lib.lib.sinkattn_plan_decode(R(q), R(k), R(v), R(bad_sinks), R(sl), 8, 0.125, _lib.PLAN_DECODE_SPLIT, buf,
                                       ctypes.byref(count))
    assert st == _lib.ERR_SHAPE and count.value == 0
    st = _lib.lib.sinkattn_plan_decode(R(q), R(k), R(v), R(s), R(sl), 8, 0.125, 5, buf, ctypes.byref(count))
    assert st == _lib.ERR_SHAPE
    st = _lib.lib.sinkattn_plan_decode(R(q), R(k), R(v), R(s), R(sl), 8, 0.125, _lib.PLAN_DECODE, None, None)
    assert st == _lib.ERR_NULL


# ----------------------------------------------------------------------------- routing and linear
def test_moe_and_linear_hand_their_sizes_to_the_launchers():
    logits, ids, w = T([1000, 128]), T([1000, 4], I32), T([1000, 4])
    take_log()
    ok(_lib.lib.sinkattn_moe_topk_softmax(R(logits), 4, 0, R(ids), R(w), None))
    (r,) = records()
    assert (r["launcher"], r["tokens"], r["experts"], r["top_k"], r["over_all"]) == ("moe_topk", 1000, 128, 4, 0)
    x, wt, bias, y = T([300, 512]), T([640, 512]), T([640], F32), T([300, 640])
    ok(_lib.lib.sinkattn_linear_bias(R(x), R(wt), R(bias), R(y), None))
    (r,) = records()
    assert (r["m"], r["n"], r["k"], r["fp8"], r["bias"]) == (300, 640, 512, False, True)


# ----------------------------------------------------------------------------- launch failure
def test_launch_failure_is_reported_with_the_runtime_message():
    q, k, v, s, sl = decode_inputs(8, 64, 8, 8192)
    po, pm, pd = T([8, 64, 8, 64], F32), T([8, 64, 8], F32), T([8, 64, 8], F32)
    take_log()
    _lib.lib.sinkattn_stub_fail_next(HIP_ERROR_INVALID_CONFIGURATION)
    st = _lib.lib.sinkattn_decode_split(R(q), R(k), R(v), R(s), R(sl), 8, 0.125, R(po), R(pm), R(pd), None)
    assert st == _lib.ERR_LAUNCH
    assert "invalid configuration" in _lib.lib.sinkattn_last_error().decode()
    records()
    ok(_lib.lib.sinkattn_decode_split(R(q), R(k), R(v), R(s), R(sl), 8, 0.125, R(po), R(pm), R(pd), None))
    assert _lib.lib.sinkattn_last_error().decode() == ""
    records()
