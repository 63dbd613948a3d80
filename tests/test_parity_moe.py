"""GPU parity of the MoE routing softmax (top-K experts, softmax over the chosen logits) against the
float64 CPU oracle, through the C ABI.

Source: "GPT-OSS on Day 0" (Perplexity): softmax after the top-K expert choice, over the K chosen
experts only; expert weights in bfloat16. Bars: expert ids bit-exact (both sides compare the same
stored logits; ties go to the lower expert index); weights within one bf16 rounding of the exact
value plus fp32 arithmetic error (relative 2^-8 + 1e-6), or 1e-6 relative for fp32 weights.
"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

BF16_W_RTOL = 2.0 ** -8 + 1e-6
F32_W_RTOL = 1e-6


def _sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_learned_softmax_amd as sa  # raises if the HIP library is missing

    return sa


def _logits(t, e, seed, dtype, scale=1.0, neg_inf_p=0.0):
    """Router logits drawn N(0, scale) (bf16 values repeat, so ties are common), optional -inf entries."""
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn((t, e), generator=g) * scale).to(dtype)
    if neg_inf_p > 0:
        x[torch.rand((t, e), generator=g) < neg_inf_p] = float("-inf")
    return x


def _check(sa, logits_cpu, k, over_all, wdtype, label, device_logits=None):
    x = device_logits if device_logits is not None else logits_cpu.cuda()
    ids, w = sa.moe_topk_softmax(x, k, over_all_experts=over_all, weights_dtype=wdtype)
    torch.cuda.synchronize()
    rids, rw = oracle.moe_topk_softmax(logits_cpu.double().numpy(), k, over_all=over_all)
    gids = ids.cpu().numpy()
    mism = int((gids != rids).sum())
    assert mism == 0, f"{label}: {mism} expert ids differ"
    gw = w.double().cpu().numpy()
    rtol = BF16_W_RTOL if wdtype == torch.bfloat16 else F32_W_RTOL
    err = np.abs(gw - rw)
    bound = rtol * np.abs(rw) + 1e-30
    worst = float(np.max(err / np.maximum(np.abs(rw), 1e-30))) if err.size else 0.0
    print(f"{label}: ids exact, worst weight rel err {worst:.2e}", flush=True)
    assert np.all(err <= bound), f"{label}: weight error above the bf16 bound"
    return gids, gw


MOE_CASES = [
    # (name, T, E, K, logits dtype, weights dtype, over_all, scale, -inf share)
    ("e128_k4_bf16", 1000, 128, 4, torch.bfloat16, torch.bfloat16, False, 1.0, 0.0),
    ("e32_k4_bf16", 1000, 32, 4, torch.bfloat16, torch.bfloat16, False, 1.0, 0.0),
    ("e256_k8_bf16", 777, 256, 8, torch.bfloat16, torch.bfloat16, False, 2.0, 0.0),
    ("e100_ragged_k6_f32w", 513, 100, 6, torch.bfloat16, torch.float32, False, 1.0, 0.0),
    ("e16_k16_f32", 300, 16, 16, torch.float32, torch.float32, False, 3.0, 0.0),
    ("e1_k1", 300, 1, 1, torch.bfloat16, torch.bfloat16, False, 1.0, 0.0),
    ("e128_f32_logits", 999, 128, 4, torch.float32, torch.bfloat16, False, 1.0, 0.0),
    ("e64_k2_over_all", 400, 64, 2, torch.bfloat16, torch.bfloat16, True, 1.0, 0.0),
    ("e200_k16_over_all_f32", 257, 200, 16, torch.float32, torch.float32, True, 2.0, 0.0),
    ("e128_neg_inf_entries", 500, 128, 8, torch.bfloat16, torch.bfloat16, False, 1.0, 0.9),
    ("e7_k5_ragged_small", 129, 7, 5, torch.bfloat16, torch.bfloat16, False, 1.0, 0.3),
    ("e128_coarse_many_ties", 1000, 128, 8, torch.bfloat16, torch.bfloat16, False, 0.01, 0.0),
]


@pytest.mark.parametrize("name,t,e,k,dt,wdt,over_all,scale,ninf", MOE_CASES, ids=[c[0] for c in MOE_CASES])
def test_moe_topk_softmax(name, t, e, k, dt, wdt, over_all, scale, ninf):
    sa = _sa()
    x = _logits(t, e, zlib.crc32(name.encode()) % 10_000, dt, scale, ninf)
    if name == "e128_coarse_many_ties":
        x = (x.float() * 100).round().div(100).to(dt)  # few distinct values per row
    _, gw = _check(sa, x, k, over_all, wdt, name)
    if not over_all and ninf == 0:
        np.testing.assert_allclose(gw.sum(axis=1), 1.0, atol=k * 2.0 ** -8)


def test_moe_rows_without_finite_logits_get_zero_weights():
    sa = _sa()
    x = _logits(64, 128, 5, torch.bfloat16)
    x[::3] = float("-inf")
    _, gw = _check(sa, x, 4, False, torch.bfloat16, "all -inf rows")
    assert np.all(gw[::3] == 0)


def test_moe_strided_logits_view():
    """Logits as a view into wider rows (e.g. a router GEMM output with padding)."""
    sa = _sa()
    buf = _logits(700, 160, 6, torch.bfloat16)
    view_cpu = buf[:, :128]
    _check(sa, view_cpu.contiguous(), 4, False, torch.bfloat16, "strided view", device_logits=buf.cuda()[:, :128])
    # rows of 132 bf16 = 264 bytes: not 16-byte aligned, so the element loads serve the full rows
    buf2 = _logits(700, 132, 8, torch.bfloat16)
    _check(sa, buf2[:, :128].contiguous(), 4, False, torch.bfloat16, "unaligned rows",
           device_logits=buf2.cuda()[:, :128])


def test_moe_full_size_65536_tokens():
    """The bench workload: 65,536 tokens x 128 experts, top-4, bf16; every row compared."""
    sa = _sa()
    x = _logits(65536, 128, 7, torch.bfloat16)
    _check(sa, x, 4, False, torch.bfloat16, "65536 x 128 top-4")
