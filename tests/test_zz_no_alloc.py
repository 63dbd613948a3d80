"""sinkattn_decode_static: the decode entry point that allocates nothing (its chunk states live in
the library's own device array), checked through the C-ABI against sinkattn_decode on a caller
workspace, which runs the same kernels. Two calls in a row, the second one smaller; a grid large
enough for the two-launch form; and replays of a captured graph (no allocation may happen under
capture) with eager work between them."""
from __future__ import annotations

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3


def _sa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import gqa_learned_softmax_amd as sa
    return sa


def _case(lens, cap, chunks, seed, hq=64, hkv=8):
    return workloads.make_decode(lens, cap, chunks, num_q_heads=hq, num_kv_heads=hkv, seed=seed, poison=True)


def _run_both(sa, case, dev):
    args = [t.to(dev) for t in (case.q, case.k, case.v, case.sinks, case.seqlens_k)]
    out_s, lse_s = sa.decode_static(*args, case.num_chunks, case.scale, return_lse=True)
    ws = sa.decode_workspace(case.q.shape[0], case.q.shape[1], case.k.shape[2], case.num_chunks, dev)
    out_w, lse_w = sa.decode_fused(*args, case.num_chunks, case.scale, ws, return_lse=True)
    torch.cuda.synchronize()
    return out_s, lse_s, out_w, lse_w


def _check(out_s, lse_s, out_w, lse_w, label):
    err = (out_s.double() - out_w.double()).abs()
    assert torch.isfinite(out_s.double()).all(), label
    assert err.max().item() <= BF16_MAX_ABS and err.mean().item() <= BF16_MEAN_ABS, (label, err.max().item())
    lerr = (lse_s - lse_w).abs()
    finite = torch.isfinite(lse_w)
    assert torch.equal(torch.isfinite(lse_s), finite), label
    assert lerr[finite].max().item() <= 1e-4 if finite.any() else True, label
    # Same kernels on the same inputs: the results agree bit for bit.
    assert torch.equal(out_s, out_w), label


def test_static_decode_two_calls_second_smaller():
    sa = _sa()
    dev = torch.device("cuda:0")
    print("static decode: 8 x 8192 keys, then 3 sequences of up to 2048 keys", flush=True)
    big = _case([8192, 8000, 1, 0, 4096, 8191, 300, 8192], 8192, 8, seed=71)
    _check(*_run_both(sa, big, dev), "first call (8 x 8192)")
    small = _case([2048, 5, 1000], 2048, 4, seed=72)
    _check(*_run_both(sa, small, dev), "second call (3 x 2048)")


def test_static_decode_two_launch_form():
    sa = _sa()
    dev = torch.device("cuda:0")
    print("static decode: 40 sequences (split + merge through the static workspace)", flush=True)
    case = _case([(i * 997) % 4096 + 1 for i in range(40)], 4096, 8, seed=73)
    _check(*_run_both(sa, case, dev), "two-launch form")


def test_static_decode_graph_replays():
    sa = _sa()
    dev = torch.device("cuda:0")
    print("static decode under graph capture, 4 replays", flush=True)
    case = _case([8192, 700, 8192, 33], 8192, 8, seed=74)
    args = [t.to(dev) for t in (case.q, case.k, case.v, case.sinks, case.seqlens_k)]
    out = torch.empty(case.q.shape, dtype=torch.bfloat16, device=dev)
    sa.decode_static(*args, case.num_chunks, case.scale, out=out)  # eager first call
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sa.decode_static(*args, case.num_chunks, case.scale, out=out)
    other = _case([100, 2000], 2048, 4, seed=75)
    for r in range(4):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r}"
        # Eager work between replays, on the same static workspace.
        o2, l2, w2, lw2 = _run_both(sa, other, dev)
        _check(o2, l2, w2, lw2, f"eager call after replay {r}")
