"""GPU parity: the HIP kernels (through the C ABI) against the float64 CPU oracle.

Both sides see the same seeded inputs (bf16 values upcast exactly for the oracle). Bars:
* bf16 inputs, fp32 accumulation: max |gpu - oracle| <= 2e-2 and mean |gpu - oracle| <= 2e-3 over
  all compared output elements;
* fp32 reference variant: ||gpu - oracle||_inf / ||oracle||_inf <= 1e-5.
Small cases compare every output element; the full-size workloads compare every output where the
oracle is cheap (decode, the long decode included) and, for prefill, every work-group tile's first
and last query position for every KV group plus random (token, head) rows.
"""
from __future__ import annotations

import math
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_REL = 1e-5


def _sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_learned_softmax_amd as sa  # raises if the HIP library is missing

    return sa


def _np(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _np32(t):
    """Exact float32 copy of a (bf16 or f32) CPU tensor, for large oracle inputs."""
    return t.detach().to("cpu", torch.float32).numpy()


def _seed(name):
    return zlib.crc32(name.encode()) % 10_000


def _dev(*ts):
    return [t.cuda() for t in ts]


def check_bf16(gpu, ref, label=""):
    g = _np(gpu)
    err = np.abs(g - ref)
    assert np.all(np.isfinite(g)), f"{label}: non-finite output"
    max_abs, mean_abs = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    print(f"{label}: max_abs={max_abs:.3e} mean_abs={mean_abs:.3e}", flush=True)
    assert max_abs <= BF16_MAX_ABS, f"{label}: max_abs {max_abs}"
    assert mean_abs <= BF16_MEAN_ABS, f"{label}: mean_abs {mean_abs}"


def check_f32(gpu, ref, label=""):
    g = _np(gpu)
    scale = float(np.abs(ref).max(initial=0.0))
    rel = float(np.abs(g - ref).max(initial=0.0)) / (scale if scale > 0 else 1.0)
    print(f"{label}: normwise rel={rel:.3e}", flush=True)
    assert rel <= F32_REL, f"{label}: rel {rel}"


def run_prefill(sa, case, out_dtype=None):
    q, k, v, sinks, cq, ck = _dev(case.q, case.k, case.v, case.sinks, case.cu_seqlens_q, case.cu_seqlens_k)
    out = sa.prefill(q, k, v, sinks, cq, ck, case.scale, case.causal, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


def oracle_prefill(case):
    return oracle.prefill(_np(case.q), _np(case.k), _np(case.v), _np(case.sinks),
                          case.cu_seqlens_q.numpy(), case.cu_seqlens_k.numpy(), case.scale, case.causal)


def oracle_decode(case):
    """Oracle decode, one sequence at a time (bounds host memory for large caches)."""
    outs, lses = [], []
    for b in range(case.q.shape[0]):
        n = int(case.seqlens_k[b])
        o, l = oracle.decode(_np(case.q[b:b + 1]), _np32(case.k[b:b + 1, :n]), _np32(case.v[b:b + 1, :n]),
                             _np(case.sinks), [n], case.scale)
        outs.append(o[0])
        lses.append(l[0])
    return np.stack(outs), np.stack(lses)


def run_decode(sa, case, return_lse=True):
    q, k, v, sinks, sl = _dev(case.q, case.k, case.v, case.sinks, case.seqlens_k)
    po, pm, pd = sa.decode_split(q, k, v, sinks, sl, case.num_chunks, case.scale)
    out, lse = sa.decode_merge(po, pm, pd, out_dtype=q.dtype, return_lse=True)
    torch.cuda.synchronize()
    return po, pm, pd, out, lse


def check_partials(po, pm, pd, case, checker, label):
    """Split-level parity: o_c and the chunk log-mass m_c + ln d_c, per chunk."""
    ro, rm, rd = oracle.decode_split(_np(case.q), _np32(case.k), _np32(case.v), _np(case.sinks),
                                     case.seqlens_k.numpy(), case.num_chunks, case.scale)
    checker(po, ro, f"{label} partial_o")
    gm, gd = _np(pm), _np(pd)
    with np.errstate(divide="ignore"):
        g_mass = np.where(gd > 0, gm + np.log(np.where(gd > 0, gd, 1.0)), -np.inf)
        r_mass = np.where(rd > 0, rm + np.log(np.where(rd > 0, rd, 1.0)), -np.inf)
    assert np.array_equal(np.isneginf(g_mass), np.isneginf(r_mass)), f"{label}: empty-chunk pattern"
    fin = np.isfinite(r_mass)
    np.testing.assert_allclose(g_mass[fin], r_mass[fin], rtol=0, atol=1e-3 if checker is check_bf16 else 1e-5)
    assert np.all(gd[~fin] == 0) and np.all(_np(po)[~fin] == 0)


# ----------------------------------------------------------------------------- tiny fp32 (C1)
def test_tiny_fp32_prefill_and_decode():
    sa = _sa()
    w = workloads.make(1)
    out = run_prefill(sa, w.prefill)
    ref, _ = oracle_prefill(w.prefill)
    check_f32(out, ref, "tiny prefill f32")

    for name, case in (("fresh", w.decode), ("last_row", w.extra["decode_last_row"])):
        po, pm, pd, dout, lse = run_decode(sa, case)
        check_partials(po, pm, pd, case, check_f32, f"tiny decode {name}")
        rout, rlse = oracle_decode(case)
        check_f32(dout, rout, f"tiny decode {name}")
        np.testing.assert_allclose(_np(lse), rlse, rtol=1e-5)
    # decode of the prefill's last row equals prefill row 127, on the GPU
    check_f32(dout[0], _np(out)[127], "tiny decode == prefill last row")


# ----------------------------------------------------------------------------- bf16 prefill, small
PREFILL_SMALL = [
    # (name, lens_q, lens_k, Hq, Hkv, causal, sink_range)
    ("one_seq_ragged", [200], None, 64, 8, True, (-2, 2)),
    ("varlen_mixed", [1, 17, 128, 129, 5, 300], None, 64, 8, True, (-2, 2)),
    ("mha_group1", [150, 33], None, 8, 8, True, (-2, 2)),
    ("group2", [97], None, 16, 8, True, (-2, 2)),
    ("group4", [211, 3], None, 16, 4, True, (-2, 2)),
    ("group16", [77, 64], None, 64, 4, True, (-2, 2)),
    ("group64", [40, 9], None, 64, 1, True, (-2, 2)),
    ("noncausal", [90, 130], None, 64, 8, False, (-2, 2)),
    ("append_lq_lt_lk", [37, 1, 64], [300, 20, 64], 64, 8, True, (-2, 2)),
    ("lq_gt_lk", [80], [50], 64, 8, True, (-2, 2)),
    ("empty_seq_in_batch", [0, 50, 0, 7], None, 64, 8, True, (-2, 2)),
    ("strong_sinks", [160], None, 64, 8, True, (25, 30)),
    ("weak_sinks", [160], None, 64, 8, True, (-30, -25)),
    ("long_tiles", [1100], None, 64, 8, True, (-4, 4)),
    ("tile_edges", [31, 32, 33, 63, 64, 65, 255, 256, 257], None, 64, 8, True, (-2, 2)),
    ("mha_long", [700], None, 4, 4, True, (-2, 2)),
    ("group128", [20, 3], None, 128, 1, True, (-2, 2)),
    ("append_long", [100], [2000], 64, 8, True, (-2, 2)),
    # More sequences than a wave has lanes: the tile search takes two and three 64-way steps.
    ("many_seqs_100", [(i * 37) % 71 for i in range(100)], None, 64, 8, True, (-2, 2)),
    ("many_seqs_4500", [(i * 7) % 5 for i in range(4500)], None, 16, 8, True, (-2, 2)),
    ("seqs_64", [(i * 29) % 40 + 1 for i in range(64)], None, 64, 8, True, (-2, 2)),
    ("seqs_65", [(i * 29) % 40 + 1 for i in range(65)], None, 64, 8, True, (-2, 2)),
]


@pytest.mark.parametrize("name,lq,lk,hq,hkv,causal,sr", PREFILL_SMALL, ids=[c[0] for c in PREFILL_SMALL])
def test_prefill_bf16_small(name, lq, lk, hq, hkv, causal, sr):
    sa = _sa()
    case = workloads.make_prefill(lq, lk, num_q_heads=hq, num_kv_heads=hkv, sink_range=sr,
                                  seed=_seed(name), causal=causal)
    out = run_prefill(sa, case)
    ref, _ = oracle_prefill(case)
    check_bf16(out, ref, f"prefill {name}")
    out32 = run_prefill(sa, case, out_dtype=torch.float32)
    check_bf16(out32, ref, f"prefill {name} f32-out")


@pytest.mark.parametrize("factor,causal", [(8.0, True), (32.0, True), (32.0, False)],
                         ids=["x8_causal", "x32_causal", "x32_noncausal"])
def test_prefill_bf16_logits_grow_after_early_keys(factor, causal):
    """Keys past the first 256 scaled by a power of two (exact in bf16): rows settle on small
    logits first, then meet logits up to ~factor times larger. x8 keeps exp2 of the logits in
    fp32 range; x32 does not, which the kernel must detect and recompute."""
    sa = _sa()
    case = workloads.make_prefill([600, 300], num_q_heads=64, num_kv_heads=8, seed=int(factor) + causal,
                                  causal=causal)
    for start, length in ((0, 600), (600, 300)):
        case.k[start + 256:start + length] *= factor
    out = run_prefill(sa, case)
    ref, _ = oracle_prefill(case)
    check_bf16(out, ref, f"prefill keys x{factor}")


# ----------------------------------------------------------------------------- split-KV prefill
PREFILL_SPLIT_CASES = [
    # (name, lens_q, lens_k, Hq, Hkv, causal, splits)
    ("append_long_kv", [100], [2000], 64, 8, True, 4),
    ("varlen_causal", [300, 77, 0, 129], None, 64, 8, True, 3),
    ("noncausal", [90, 130], None, 64, 8, False, 5),
    ("more_splits_than_tiles", [70], [300], 64, 8, True, 40),
    ("one_split", [200], None, 64, 8, True, 1),
    ("group16_append", [33, 5], [700, 64], 64, 4, True, 6),
    ("many_seqs", [(i * 13) % 40 for i in range(130)], [(i * 13) % 40 + 50 for i in range(130)], 64, 8, True, 3),
]


def _check_split_states(po, pm, pd, rpo, rpm, rpd, label):
    """States are unique up to their reference logit: compare o and m + ln d (the log-weight).
    The prefill row sum is taken on bf16-rounded P (relative error <= 2^-9 per term), so the
    log-weight is compared to 5e-3."""
    gpo, gpm, gpd = _np(po), _np(pm), _np(pd)
    ref_live, live = rpd > 0, gpd > 0
    assert np.array_equal(ref_live, live), f"{label}: empty splits differ"
    assert np.all(np.isneginf(gpm[~live])), f"{label}: empty split with finite m"
    lw, rlw = gpm[live] + np.log(gpd[live]), rpm[ref_live] + np.log(rpd[ref_live])
    np.testing.assert_allclose(lw, rlw, atol=5e-3, err_msg=f"{label}: log-weight")
    check_bf16(torch.from_numpy(np.where(live[..., None], gpo, 0.0)),
               np.where(ref_live[..., None], rpo, 0.0), f"{label} o")


@pytest.mark.parametrize("name,lq,lk,hq,hkv,causal,splits", PREFILL_SPLIT_CASES,
                         ids=[c[0] for c in PREFILL_SPLIT_CASES])
def test_prefill_split_bf16(name, lq, lk, hq, hkv, causal, splits):
    sa = _sa()
    case = workloads.make_prefill(lq, lk, num_q_heads=hq, num_kv_heads=hkv, seed=_seed(name), causal=causal)
    q, k, v, sinks, cq, ck = _dev(case.q, case.k, case.v, case.sinks, case.cu_seqlens_q, case.cu_seqlens_k)
    po, pm, pd = sa.prefill_split(q, k, v, sinks, cq, ck, case.scale, causal, splits)
    torch.cuda.synchronize()
    rpo, rpm, rpd = oracle.prefill_split(_np(case.q), _np(case.k), _np(case.v), _np(case.sinks),
                                         case.cu_seqlens_q.numpy(), case.cu_seqlens_k.numpy(), case.scale,
                                         causal, splits)
    _check_split_states(po, pm, pd, rpo, rpm, rpd, f"prefill_split {name}")
    out = sa.prefill_kv_split(q, k, v, sinks, cq, ck, case.scale, causal, splits)
    torch.cuda.synchronize()
    ref, _ = oracle_prefill(case)
    check_bf16(out, ref, f"prefill_kv_split {name}")


def test_prefill_split_logits_overflow_recompute():
    """Later keys x32: zero-reference tiles overflow, the work-group recomputes; per split too."""
    sa = _sa()
    case = workloads.make_prefill([300], [1200], num_q_heads=64, num_kv_heads=8, seed=77)
    case.k[256:] *= 32.0
    q, k, v, sinks, cq, ck = _dev(case.q, case.k, case.v, case.sinks, case.cu_seqlens_q, case.cu_seqlens_k)
    out = sa.prefill_kv_split(q, k, v, sinks, cq, ck, case.scale, True, 3)
    torch.cuda.synchronize()
    ref, _ = oracle_prefill(case)
    check_bf16(out, ref, "prefill_kv_split keys x32")


def test_prefill_split_fp32_tiny():
    sa = _sa()
    pre = workloads.make(1).prefill
    q, k, v, sinks, cq, ck = _dev(pre.q, pre.k, pre.v, pre.sinks, pre.cu_seqlens_q, pre.cu_seqlens_k)
    po, pm, pd = sa.prefill_split(q, k, v, sinks, cq, ck, pre.scale, True, 3)
    torch.cuda.synchronize()
    rpo, rpm, rpd = oracle.prefill_split(_np(pre.q), _np(pre.k), _np(pre.v), _np(pre.sinks),
                                         pre.cu_seqlens_q.numpy(), pre.cu_seqlens_k.numpy(), pre.scale, True, 3)
    gpd = _np(pd)
    assert np.array_equal(gpd > 0, rpd > 0)
    live = rpd > 0
    np.testing.assert_allclose(_np(pm)[live] + np.log(gpd[live]), rpm[live] + np.log(rpd[live]), rtol=1e-6)
    out = sa.prefill_kv_split(q, k, v, sinks, cq, ck, pre.scale, True, 3)
    torch.cuda.synchronize()
    ref, _ = oracle_prefill(pre)
    check_f32(out, ref, "prefill_kv_split tiny f32")


def test_prefill_split_append_32k_sampled_rows():
    """Chunked prefill of 512 new tokens against a 32768-key cache (64/8 heads), 8 splits:
    sampled rows against the oracle row by row."""
    sa = _sa()
    case = workloads.make_prefill([512], [32768], num_q_heads=64, num_kv_heads=8, seed=4321)
    q, k, v, sinks, cq, ck = _dev(case.q, case.k, case.v, case.sinks, case.cu_seqlens_q, case.cu_seqlens_k)
    out = sa.prefill_kv_split(q, k, v, sinks, cq, ck, case.scale, True, 8)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    tokens = np.concatenate([[0, 511], rng.integers(0, 512, 14)])
    heads = rng.integers(0, 64, tokens.size)
    ref, _ = oracle.prefill_at(_np(case.q), _np(case.k), _np(case.v), _np(case.sinks), case.cu_seqlens_q.numpy(),
                               case.cu_seqlens_k.numpy(), case.scale, True, tokens, heads)
    got = torch.from_numpy(_np(out)[tokens, heads])
    check_bf16(got, ref, "prefill_kv_split append 512 x 32768 (sampled)")


def test_prefill_bf16_sink_neg_inf_is_plain_attention():
    sa = _sa()
    case = workloads.make_prefill([130, 64], num_q_heads=64, num_kv_heads=8, seed=7)
    case.sinks[:] = float("-inf")
    out = run_prefill(sa, case)
    ref, _ = oracle_prefill(case)
    check_bf16(out, ref, "prefill sink=-inf")


def test_prefill_bf16_strided_views():
    """q/k/v as views into one fused [T, Hq + 2 Hkv, D] buffer; out with padded head stride."""
    sa = _sa()
    case = workloads.make_prefill([150], num_q_heads=64, num_kv_heads=8, seed=11)
    fused = torch.cat([case.q, case.k, case.v], dim=1).cuda()
    q, k, v = fused[:, :64], fused[:, 64:72], fused[:, 72:80]
    out_buf = torch.zeros(150, 64, 72, dtype=torch.bfloat16, device="cuda")
    out = out_buf[:, :, :64]
    sinks, cq, ck = _dev(case.sinks, case.cu_seqlens_q, case.cu_seqlens_k)
    sa.prefill(q, k, v, sinks, cq, ck, case.scale, True, out=out)
    torch.cuda.synchronize()
    ref, _ = oracle_prefill(case)
    check_bf16(out, ref, "prefill strided")
    assert torch.all(out_buf[:, :, 64:] == 0), "padding between output rows was written"


# ----------------------------------------------------------------------------- bf16 decode, small
DECODE_SMALL = [
    # (name, lens, cap, chunks, Hq, Hkv, sink_range, outlier_p)
    ("uniform", [512, 512], 512, 4, 64, 8, (-2, 2), 0.0),
    ("ragged_empty_chunks", [1, 0, 33, 700, 1023, 64], 1024, 8, 64, 8, (-2, 2), 0.0),
    ("one_chunk", [300, 5], 320, 1, 64, 8, (-2, 2), 0.0),
    ("many_chunks", [257, 100], 257, 40, 64, 8, (-2, 2), 0.0),
    ("group1", [200, 31], 256, 4, 8, 8, (-2, 2), 0.0),
    ("group2", [150], 160, 3, 16, 8, (-2, 2), 0.0),
    ("group4", [99, 300], 300, 2, 16, 4, (-2, 2), 0.0),
    ("group16", [333], 400, 5, 64, 4, (-2, 2), 0.0),
    ("outliers", [2000, 1500], 2048, 2, 64, 8, (-4, 4), 0.02),
    ("strong_sinks", [128, 64], 128, 2, 64, 8, (25, 30), 0.0),
    ("weak_sinks", [128, 64], 128, 2, 64, 8, (-30, -25), 0.0),
    ("kv_len_1", [1, 1, 1], 16, 4, 64, 8, (-2, 2), 0.0),
    ("odd_kv_heads", [300, 77], 320, 4, 12, 3, (-2, 2), 0.0),
    # B * Hkv/2 * C = 256 with a token-major cache: the two-KV-heads-per-work-group kernel
    ("paired_heads", [250, 3, 0, 129], 256, 16, 64, 8, (-2, 2), 0.0),
    # 8 x 4 x 8 = 256 paired work-groups of 1024-key chunks: one round, so each wave stages its own
    # keys' rows (private staging); lengths end inside blocks, on block borders and at zero
    ("paired_private_ragged", [8191, 4097, 1, 0, 2048, 6000, 63, 65], 8192, 8, 64, 8, (-2, 2), 0.0),
    ("single_kv_head", [500, 64], 512, 3, 16, 1, (-2, 2), 0.0),
    # B * Hkv/4 * C = 512 with a token-major cache: the four-KV-heads-per-work-group kernel
    ("quad_heads", [(37 * i) % 513 for i in range(32)], 512, 8, 64, 8, (-2, 2), 0.0),
    # 1 x 8 x 20 = 160 work-groups: one round, so sinkattn_decode merges more than 16 chunks in its tail
    ("many_chunks_one_round", [1000], 1024, 20, 64, 8, (-2, 2), 0.0),
    # More than one round of work-groups, whose (sequence, head set) index is rotated by the chunk,
    # with 12 and 15 rows per chunk (not multiples of the eight XCDs)
    ("rotated_paired_r12", [900, 17, 480], 960, 30, 64, 8, (-2, 2), 0.0),
    ("rotated_single_r15", [300, 0, 77, 299, 150], 320, 20, 12, 3, (-2, 2), 0.0),
]


@pytest.mark.parametrize("name,lens,cap,chunks,hq,hkv,sr,op", DECODE_SMALL, ids=[c[0] for c in DECODE_SMALL])
def test_decode_bf16_small(name, lens, cap, chunks, hq, hkv, sr, op):
    sa = _sa()
    # rows past each length are NaN: reading any of them would poison the output
    case = workloads.make_decode(lens, cap, chunks, num_q_heads=hq, num_kv_heads=hkv, sink_range=sr,
                                 outlier_p=op, seed=_seed(name), poison=True)
    po, pm, pd, out, lse = run_decode(sa, case)
    check_partials(po, pm, pd, case, check_bf16, f"decode {name}")
    ref, rlse = oracle_decode(case)
    check_bf16(out, ref, f"decode {name}")
    np.testing.assert_allclose(_np(lse), rlse, rtol=0, atol=1e-3)


def test_decode_bf16_sink_neg_inf_and_zero_length():
    sa = _sa()
    case = workloads.make_decode([0, 40, 0], 64, 4, seed=5, poison=True)
    case.sinks[::2] = float("-inf")
    po, pm, pd, out, lse = run_decode(sa, case)
    check_partials(po, pm, pd, case, check_bf16, "decode -inf sinks")
    ref, rlse = oracle_decode(case)
    check_bf16(out, ref, "decode -inf sinks")
    g = _np(lse)
    assert np.array_equal(np.isneginf(g), np.isneginf(rlse))
    fin = np.isfinite(rlse)
    np.testing.assert_allclose(g[fin], rlse[fin], atol=1e-3)
    assert torch.all(out[0] == 0) and torch.all(out[2] == 0)


def test_decode_equals_prefill_last_row_bf16():
    """Decode of a sequence's last query row equals that row of causal prefill (on the GPU)."""
    sa = _sa()
    case = workloads.make_prefill([333], num_q_heads=64, num_kv_heads=8, seed=3)
    pre = run_prefill(sa, case, out_dtype=torch.float32)
    dec = workloads.DecodeCase(case.q[332:333].clone(), case.k.reshape(1, 333, 8, 64).clone(),
                               case.v.reshape(1, 333, 8, 64).clone(), case.sinks.clone(),
                               torch.tensor([333], dtype=torch.int32), 3)
    _, _, _, out, _ = run_decode(sa, dec)
    check_bf16(out[0], _np(pre)[332], "decode vs prefill last row")


# ----------------------------------------------------------------------------- full-size workloads
def test_full_decode_workload_2():
    sa = _sa()
    case = workloads.make(2, poison=True).decode
    po, pm, pd, out, lse = run_decode(sa, case)
    ref, rlse = oracle_decode(case)
    check_bf16(out, ref, "workload 2 decode")
    np.testing.assert_allclose(_np(lse), rlse, atol=1e-3)


def _decode_rows(case, pairs):
    """Oracle decode for selected (b, kv-head) groups; returns {(b, g): (out [G, D], lse [G])}."""
    group = case.q.shape[1] // case.k.shape[2]
    res = {}
    for b, g in pairs:
        q = _np(case.q[b:b + 1, g * group:(g + 1) * group])
        n = int(case.seqlens_k[b])
        k = _np(case.k[b:b + 1, :n, g:g + 1])
        v = _np(case.v[b:b + 1, :n, g:g + 1])
        out, lse = oracle.decode(q, k, v, _np(case.sinks[g * group:(g + 1) * group]), [n], case.scale)
        res[(b, g)] = (out[0], lse[0])
    return res


def test_full_long_decode_workload_4_all_groups():
    """Every (sequence, KV-head) group of the long decode: all 32 x 8 groups, output and lse."""
    sa = _sa()
    case = workloads.make(4, poison=True).decode
    _, _, _, out, lse = run_decode(sa, case)
    pairs = [(b, g) for b in range(case.q.shape[0]) for g in range(case.k.shape[2])]
    ref = _decode_rows(case, pairs)
    group = case.q.shape[1] // case.k.shape[2]
    g_out = np.stack([_np(out[b, g * group:(g + 1) * group]) for b, g in pairs])
    r_out = np.stack([ref[p][0] for p in pairs])
    check_bf16(torch.from_numpy(g_out), r_out, "workload 4 decode (all 256 groups)")
    g_lse = np.stack([_np(lse[b, g * group:(g + 1) * group]) for b, g in pairs])
    r_lse = np.stack([ref[p][1] for p in pairs])
    np.testing.assert_allclose(g_lse, r_lse, atol=1e-3)


def _stratified_rows(case, n_random, seed):
    """(token, head) rows to check at full size: for every work-group query tile (32 consecutive
    positions of one sequence, which the kernel runs for the 8 heads of one KV group) its first
    and its last position, once for each KV group, the head within the group rotating from tile
    to tile; plus ``n_random`` uniformly drawn rows. That reaches every tile, the diagonal tiles
    where the causal mask cuts through, and every tile's first and last wave."""
    tile_positions = 32
    h_q, h_kv = case.q.shape[1], case.k.shape[1]
    group = h_q // h_kv
    tokens, heads = [], []
    cu = case.cu_seqlens_q.tolist()
    tile_index = 0
    for b in range(len(cu) - 1):
        for start in range(cu[b], cu[b + 1], tile_positions):
            last = min(start + tile_positions, cu[b + 1]) - 1
            for j, t in enumerate((start, last)):
                for g in range(h_kv):
                    tokens.append(t)
                    heads.append(g * group + (tile_index + 3 * j + g) % group)
            tile_index += 1
    rng = np.random.default_rng(seed)
    tokens += rng.integers(0, case.q.shape[0], n_random).tolist()
    heads += rng.integers(0, h_q, n_random).tolist()
    return np.array(tokens), np.array(heads)


def _stratified_prefill(sa, case, n_random, seed, label):
    out = run_prefill(sa, case)
    tokens, heads = _stratified_rows(case, n_random, seed)
    ref, _ = oracle.prefill_at(_np(case.q), _np(case.k), _np(case.v), _np(case.sinks), case.cu_seqlens_q.numpy(),
                               case.cu_seqlens_k.numpy(), case.scale, case.causal, tokens, heads)
    g = out[torch.from_numpy(tokens).cuda(), torch.from_numpy(heads).cuda()]
    check_bf16(g, ref, f"{label} ({len(tokens)} rows)")


def test_full_prefill_workload_3_stratified():
    sa = _sa()
    case = workloads.make(3).prefill
    _stratified_prefill(sa, case, 400, 3, "workload 3 prefill (every tile's first and last row)")


def test_full_mixed_workload_5():
    sa = _sa()
    w = workloads.make(5, poison=True)
    po, pm, pd, out, lse = run_decode(sa, w.decode)
    ref, rlse = oracle_decode(w.decode)
    check_bf16(out, ref, "workload 5 decode")
    _stratified_prefill(sa, w.prefill, 400, 5, "workload 5 prefill (every tile's first and last row)")


def test_graph_replays_match_eager():
    """The kernels captured in a HIP graph give the eager result on every replay."""
    sa = _sa()
    dec = workloads.make_decode([700, 33, 1024, 0], 1024, 8, seed=21)
    pre = workloads.make_prefill([300, 77], seed=22)
    q, k, v, s, sl = _dev(dec.q, dec.k, dec.v, dec.sinks, dec.seqlens_k)
    pq, pk, pv, ps, cq, ck = _dev(pre.q, pre.k, pre.v, pre.sinks, pre.cu_seqlens_q, pre.cu_seqlens_k)
    po = torch.empty((4, 64, 8, 64), dtype=torch.float32, device="cuda")
    pm = torch.empty((4, 64, 8), dtype=torch.float32, device="cuda")
    pd = torch.empty((4, 64, 8), dtype=torch.float32, device="cuda")
    out = torch.empty((4, 64, 64), dtype=torch.bfloat16, device="cuda")
    pout = torch.empty_like(pq)

    def work():
        sa.decode_split(q, k, v, s, sl, 8, dec.scale, po, pm, pd)
        sa.decode_merge(po, pm, pd, out=out)
        sa.prefill(pq, pk, pv, ps, cq, ck, pre.scale, True, out=pout)

    work()
    torch.cuda.synchronize()
    eager_dec, eager_pre = out.clone(), pout.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    for rep in range(4):
        out.zero_()
        pout.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_dec), f"decode differs on replay {rep}"
        assert torch.equal(pout, eager_pre), f"prefill differs on replay {rep}"
        work()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager_dec)


# ----------------------------------------------------------------------------- merge on many rows
@pytest.mark.parametrize("chunks", [1, 3, 8, 16, 17])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_merge_many_rows_random_states(chunks, out_dtype):
    """Merge of 8412 rows (701 x 12 heads: not a multiple of the 16 rows a four-row-per-wave
    work-group takes) of random chunk states with empty chunks and fully empty rows, against the
    oracle's merge. Up to 16 chunks this is the four-rows-per-wave kernel; 17 takes one wave per row."""
    sa = _sa()
    gen = torch.Generator().manual_seed(_seed(f"merge_many_{chunks}"))
    b, h, dim = 701, 12, 64
    po = torch.randn((b, h, chunks, dim), generator=gen, dtype=torch.float32)
    pm = (torch.rand((b, h, chunks), generator=gen) * 10.0 - 5.0).float()
    pd = (torch.rand((b, h, chunks), generator=gen) * 1.5 + 0.5).float()
    empty = torch.rand((b, h, chunks), generator=gen) < 0.2
    empty[::7] = True  # every seventh sequence: all of its rows have no key at all
    pm[empty] = float("-inf")
    pd[empty] = 0.0
    po[empty] = 0.0
    ref, rlse = oracle.merge(po.double().numpy(), pm.double().numpy(), pd.double().numpy())
    gpo, gpm, gpd = _dev(po, pm, pd)
    out, lse = sa.decode_merge(gpo, gpm, gpd, out_dtype=out_dtype, return_lse=True)
    torch.cuda.synchronize()
    label = f"merge {b * h} rows x {chunks} chunks {out_dtype}"
    (check_bf16 if out_dtype == torch.bfloat16 else check_f32)(out, ref, label)
    g = _np(lse)
    assert np.array_equal(np.isneginf(g), np.isneginf(rlse)), label
    fin = np.isfinite(rlse)
    np.testing.assert_allclose(g[fin], rlse[fin], rtol=0, atol=1e-4)


# ----------------------------------------------------------------------------- fused split + merge
FUSED_CASES = [c for c in DECODE_SMALL if c[0] in
               ("uniform", "ragged_empty_chunks", "many_chunks", "group16", "outliers", "odd_kv_heads",
                "single_kv_head", "paired_heads", "paired_private_ragged", "quad_heads", "kv_len_1", "weak_sinks",
                "many_chunks_one_round")]


@pytest.mark.parametrize("name,lens,cap,chunks,hq,hkv,sr,op", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_decode_fused_bf16(name, lens, cap, chunks, hq, hkv, sr, op):
    sa = _sa()
    case = workloads.make_decode(lens, cap, chunks, num_q_heads=hq, num_kv_heads=hkv, sink_range=sr,
                                 outlier_p=op, seed=_seed(name), poison=True)
    q, k, v, sinks, sl = _dev(case.q, case.k, case.v, case.sinks, case.seqlens_k)
    ws = sa.decode_workspace(len(lens), hq, hkv, chunks, "cuda")
    ref, rlse = oracle_decode(case)
    for call in range(2):  # the second call reuses the workspace the first left behind
        out, lse = sa.decode_fused(q, k, v, sinks, sl, chunks, case.scale, ws, return_lse=True)
        torch.cuda.synchronize()
        check_bf16(out, ref, f"fused {name} call {call}")
        g = _np(lse)
        assert np.array_equal(np.isneginf(g), np.isneginf(rlse))
        fin = np.isfinite(rlse)
        np.testing.assert_allclose(g[fin], rlse[fin], atol=1e-3)
    counter_bytes = sa._lib.lib.sinkattn_decode_workspace_counter_bytes(len(lens), hkv)
    assert torch.count_nonzero(ws[:counter_bytes]).item() == 0, "counters not reset"


def _head_major(t):
    """A [B, Lcap, Hkv, D] cache stored head-major ([B, Hkv, Lcap, D] memory), seen through strides."""
    return t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)


# one-round single-head grid (8 x 8 x 4 = 256 work-groups: the single launch), a multi-round one
# (16 x 8 x 4 = 512: split then merge), and ragged lengths with empty chunks
@pytest.mark.parametrize("lens,chunks", [([700, 33, 1024, 0, 513, 1, 64, 999], 4),
                                         ([700, 33, 1024, 0, 513, 1, 64, 999] * 2, 4),
                                         ([1, 0, 333, 1024], 7)], ids=["one_round", "two_rounds", "ragged"])
def test_decode_head_major_cache(lens, chunks):
    sa = _sa()
    case = workloads.make_decode(lens, 1024, chunks, seed=_seed(f"head_major_{len(lens)}_{chunks}"), poison=True)
    q, sinks, sl = _dev(case.q, case.sinks, case.seqlens_k)
    k, v = _head_major(case.k.cuda()), _head_major(case.v.cuda())
    assert k.stride(2) == 1024 * 64 and not k.is_contiguous()
    ref, rlse = oracle_decode(case)
    po, pm, pd = sa.decode_split(q, k, v, sinks, sl, chunks, case.scale)
    out, lse = sa.decode_merge(po, pm, pd, out_dtype=q.dtype, return_lse=True)
    torch.cuda.synchronize()
    check_partials(po, pm, pd, case, check_bf16, "head-major split")
    check_bf16(out, ref, "head-major split + merge")
    ws = sa.decode_workspace(len(lens), 64, 8, chunks, "cuda")
    for call in range(2):
        fout, flse = sa.decode_fused(q, k, v, sinks, sl, chunks, case.scale, ws, return_lse=True)
        torch.cuda.synchronize()
        check_bf16(fout, ref, f"head-major sinkattn_decode call {call}")
        g = _np(flse)
        assert np.array_equal(np.isneginf(g), np.isneginf(rlse))
        fin = np.isfinite(rlse)
        np.testing.assert_allclose(g[fin], rlse[fin], atol=1e-3)


def test_decode_multi_head_major_cache():
    sa = _sa()
    case = workloads.make_decode([300, 77, 5, 1000], 1024, 4, seed=_seed("head_major_multi"), poison=True, q_len=4)
    q, sinks, sl = _dev(case.q, case.sinks, case.seqlens_k)
    k, v = _head_major(case.k.cuda()), _head_major(case.v.cuda())
    po, pm, pd = sa.decode_multi_split(q, k, v, sinks, sl, 4, case.scale)
    out = sa.decode_merge(po, pm, pd, out_dtype=q.dtype)
    torch.cuda.synchronize()
    check_multi_partials(po, pm, pd, case, check_bf16, "head-major multi split")
    ref, _ = oracle_decode_multi(case)
    check_bf16(out.view(4, 4, 64, 64), ref, "head-major multi")


def test_decode_fused_workspace_reuse_with_smaller_problem():
    """A workspace sized for a large call serves a smaller, different call next."""
    sa = _sa()
    big = workloads.make_decode([900, 1024, 5, 700, 1, 0, 333, 1000], 1024, 8, seed=31, poison=True)
    small = workloads.make_decode([77, 3], 128, 4, num_q_heads=16, num_kv_heads=2, seed=32, poison=True)
    ws = sa.decode_workspace(8, 64, 8, 8, "cuda")
    for case in (big, small, big):
        q, k, v, sinks, sl = _dev(case.q, case.k, case.v, case.sinks, case.seqlens_k)
        out = sa.decode_fused(q, k, v, sinks, sl, case.num_chunks, case.scale, ws)
        torch.cuda.synchronize()
        ref, _ = oracle_decode(case)
        check_bf16(out, ref, f"fused reuse B={case.q.shape[0]}")
    assert torch.count_nonzero(ws[:sa._lib.lib.sinkattn_decode_workspace_counter_bytes(8, 8)]).item() == 0


def test_decode_fused_fp32_tiny():
    sa = _sa()
    w = workloads.make(1)
    case = w.decode
    q, k, v, sinks, sl = _dev(case.q, case.k, case.v, case.sinks, case.seqlens_k)
    ws = sa.decode_workspace(1, 4, 1, 4, "cuda")
    out, lse = sa.decode_fused(q, k, v, sinks, sl, 4, case.scale, ws, return_lse=True)
    torch.cuda.synchronize()
    ref, rlse = oracle_decode(case)
    check_f32(out, ref, "fused tiny f32")
    np.testing.assert_allclose(_np(lse), rlse, rtol=1e-5)


def test_full_decode_workload_2_fused():
    sa = _sa()
    case = workloads.make(2, poison=True).decode
    q, k, v, sinks, sl = _dev(case.q, case.k, case.v, case.sinks, case.seqlens_k)
    ws = sa.decode_workspace(8, 64, 8, 8, "cuda")
    out = sa.decode_fused(q, k, v, sinks, sl, 8, case.scale, ws)
    torch.cuda.synchronize()
    ref, _ = oracle_decode(case)
    check_bf16(out, ref, "workload 2 fused decode")


def test_fused_decode_workspace_shared_by_both_forms():
    """One workspace serves a long grid (split then merge), then a one-round grid (single launch with
    arrival counters), then the long grid again: the counters must still be zero when the single
    launch needs them, and its partials must not leak into the next call."""
    sa = _sa()
    long_case = workloads.make_decode([700, 33, 1024, 0] * 16, 1024, 8, seed=43)  # 64 x 2 x 8 quads
    short_case = workloads.make_decode([1000, 5, 512, 1024, 77, 0, 300, 999], 1024, 8, seed=44)  # 8 x 4 x 8 pairs
    ws = sa.decode_workspace(64, 64, 8, 8, "cuda")
    for name, case in (("long", long_case), ("short", short_case), ("short again", short_case),
                       ("long again", long_case)):
        q, k, v, s, sl = _dev(case.q, case.k, case.v, case.sinks, case.seqlens_k)
        out, lse = sa.decode_fused(q, k, v, s, sl, 8, case.scale, ws, return_lse=True)
        torch.cuda.synchronize()
        ref, rlse = oracle_decode(case)
        check_bf16(out, ref, f"shared workspace, {name}")
        g = _np(lse)
        assert np.array_equal(np.isneginf(g), np.isneginf(rlse))
        fin = np.isfinite(rlse)
        np.testing.assert_allclose(g[fin], rlse[fin], atol=1e-3)


# 2 x 4 x 8 = 64 work-groups per copy of the lengths: two copies are one round of pairs (the single
# launch with its arrival counters), sixteen copies are eight rounds (split then merge)
@pytest.mark.parametrize("copies", [2, 16], ids=["one_launch", "split_then_merge"])
def test_graph_replays_fused_decode(copies):
    sa = _sa()
    dec = workloads.make_decode([700, 33, 1024, 0] * copies, 1024, 8, seed=41)
    q, k, v, s, sl = _dev(dec.q, dec.k, dec.v, dec.sinks, dec.seqlens_k)
    b = 4 * copies
    ws = sa.decode_workspace(b, 64, 8, 8, "cuda")
    out = torch.empty((b, 64, 64), dtype=torch.bfloat16, device="cuda")
    sa.decode_fused(q, k, v, s, sl, 8, dec.scale, ws, out=out)
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sa.decode_fused(q, k, v, s, sl, 8, dec.scale, ws, out=out)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sa.decode_fused(q, k, v, s, sl, 8, dec.scale, ws, out=out)
    for rep in range(4):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
        sa.decode_fused(q, k, v, s, sl, 8, dec.scale, ws, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


# ----------------------------------------------------------------------------- multi-token decode
def oracle_decode_multi(case):
    """Oracle multi-token decode, one sequence at a time."""
    outs, lses = [], []
    for b in range(case.q.shape[0]):
        n = int(case.seqlens_k[b])
        o, l = oracle.decode_multi(_np(case.q[b:b + 1]), _np32(case.k[b:b + 1, :n]), _np32(case.v[b:b + 1, :n]),
                                   _np(case.sinks), [n], case.scale)
        outs.append(o[0])
        lses.append(l[0])
    return np.stack(outs), np.stack(lses)


def check_multi_partials(po, pm, pd, case, checker, label):
    """Chunk-level parity per (b, t, h, c): o_c and the chunk log-mass m_c + ln d_c."""
    ro, rm, rd = oracle.decode_multi_split(_np(case.q), _np32(case.k), _np32(case.v), _np(case.sinks),
                                           case.seqlens_k.numpy(), case.num_chunks, case.scale)
    checker(po, ro, f"{label} partial_o")
    gm, gd = _np(pm), _np(pd)
    with np.errstate(divide="ignore"):
        g_mass = np.where(gd > 0, gm + np.log(np.where(gd > 0, gd, 1.0)), -np.inf)
        r_mass = np.where(rd > 0, rm + np.log(np.where(rd > 0, rd, 1.0)), -np.inf)
    assert np.array_equal(np.isneginf(g_mass), np.isneginf(r_mass)), f"{label}: empty-chunk pattern"
    fin = np.isfinite(r_mass)
    np.testing.assert_allclose(g_mass[fin], r_mass[fin], rtol=0, atol=1e-3 if checker is check_bf16 else 1e-5)
    assert np.all(gd[~fin] == 0) and np.all(_np(po)[~fin] == 0)


MULTI_CASES = [
    # (name, lens, cap, chunks, Hq, Hkv, T): G x T query rows per KV head in 16-column tiles
    ("t2_uniform", [512, 512], 512, 4, 64, 8, 2),                     # 16 rows, one tile
    ("t3_partial_tile", [300, 77, 5], 320, 4, 64, 8, 3),              # 24 rows, two tiles
    ("t4_ragged_short", [1, 0, 33, 700, 1023, 64], 1024, 8, 64, 8, 4),  # lengths below T
    ("t5_three_tiles", [450, 129], 512, 4, 64, 8, 5),                 # 40 rows
    ("t7_four_tiles", [260, 64, 3], 320, 5, 64, 8, 7),                # 56 rows
    ("t8_four_tiles", [1000, 517, 8, 9], 1024, 8, 64, 8, 8),          # 64 rows
    ("t8_mask_straddles_chunk", [130, 131], 192, 3, 64, 8, 8),        # masked keys on both sides of 128
    ("t8_many_chunks", [257, 100], 257, 40, 64, 8, 8),
    ("t2_group16", [333, 40], 400, 5, 64, 4, 2),                      # 32 rows
    ("t4_group16", [333, 40], 400, 5, 64, 4, 4),                      # 64 rows
    ("t8_group1", [200, 31], 256, 4, 8, 8, 8),                        # 8 rows
    ("t6_group2", [150, 6], 160, 3, 16, 8, 6),                        # 12 rows
    ("t3_odd_kv_heads", [300, 77], 320, 4, 12, 3, 3),
    ("t2_paired_heads", [250, 3, 0, 129], 256, 16, 64, 8, 2),         # paired-head work-groups
    ("t4_paired_heads", [250, 3, 0, 129], 256, 16, 64, 8, 4),
    # 8 x 4 x 8 = 256 paired work-groups: one round, private staging, lengths at and below T
    ("t2_private_ragged", [8191, 1, 0, 2, 4097, 65, 64, 6000], 8192, 8, 64, 8, 2),
    ("t2_quad_heads", [4 + (37 * i) % 509 for i in range(32)], 512, 8, 64, 8, 2),   # four-head work-groups
    ("t4_quad_heads", [4 + (37 * i) % 509 for i in range(32)], 512, 8, 64, 8, 4),
    ("t1_is_decode", [700, 5], 768, 4, 64, 8, 1),
    ("t4_many_chunks_one_round", [1000], 1024, 20, 64, 8, 4),        # single launch, 20 chunks
]


@pytest.mark.parametrize("name,lens,cap,chunks,hq,hkv,t", MULTI_CASES, ids=[c[0] for c in MULTI_CASES])
def test_decode_multi_bf16(name, lens, cap, chunks, hq, hkv, t):
    sa = _sa()
    case = workloads.make_decode(lens, cap, chunks, num_q_heads=hq, num_kv_heads=hkv, seed=_seed(name),
                                 poison=True, q_len=t)
    q, k, v, sinks, sl = _dev(case.q, case.k, case.v, case.sinks, case.seqlens_k)
    po, pm, pd = sa.decode_multi_split(q, k, v, sinks, sl, chunks, case.scale)
    out, lse = sa.decode_merge(po, pm, pd, out_dtype=q.dtype, return_lse=True)
    torch.cuda.synchronize()
    check_multi_partials(po, pm, pd, case, check_bf16, f"multi {name}")
    ref, rlse = oracle_decode_multi(case)
    b = len(lens)
    check_bf16(out.view(b, t, hq, 64), ref, f"multi {name}")
    g = _np(lse).reshape(rlse.shape)
    assert np.array_equal(np.isneginf(g), np.isneginf(rlse))
    fin = np.isfinite(rlse)
    np.testing.assert_allclose(g[fin], rlse[fin], rtol=0, atol=1e-3)
    if t == 1:  # the single-token entry point computes the same partials
        so, sm, sd = sa.decode_split(q[:, 0], k, v, sinks, sl, chunks, case.scale)
        torch.cuda.synchronize()
        assert torch.equal(so, po) and torch.equal(sm, pm) and torch.equal(sd, pd)


@pytest.mark.parametrize("name,lens,cap,chunks,hq,hkv,t",
                         [c for c in MULTI_CASES if c[0] in ("t3_partial_tile", "t4_ragged_short", "t8_four_tiles",
                                                             "t4_paired_heads", "t2_quad_heads", "t4_quad_heads",
                                                             "t6_group2", "t4_many_chunks_one_round",
                                                             "t2_private_ragged")],
                         ids=lambda x: x if isinstance(x, str) else None)
def test_decode_multi_fused_bf16(name, lens, cap, chunks, hq, hkv, t):
    sa = _sa()
    case = workloads.make_decode(lens, cap, chunks, num_q_heads=hq, num_kv_heads=hkv, seed=_seed(name),
                                 poison=True, q_len=t)
    q, k, v, sinks, sl = _dev(case.q, case.k, case.v, case.sinks, case.seqlens_k)
    b = len(lens)
    ws = sa.decode_workspace(b * t, hq, hkv, chunks, "cuda")
    ref, rlse = oracle_decode_multi(case)
    for call in range(2):  # the second call reuses the workspace the first left behind
        out, lse = sa.decode_multi_fused(q, k, v, sinks, sl, chunks, case.scale, ws, return_lse=True)
        torch.cuda.synchronize()
        check_bf16(out, ref, f"multi fused {name} call {call}")
        g = _np(lse)
        assert np.array_equal(np.isneginf(g), np.isneginf(rlse))
        fin = np.isfinite(rlse)
        np.testing.assert_allclose(g[fin], rlse[fin], atol=1e-3)
    counter_bytes = sa._lib.lib.sinkattn_decode_workspace_counter_bytes(b * t, hkv)
    assert torch.count_nonzero(ws[:counter_bytes]).item() == 0, "counters not reset"


def test_decode_multi_strided_query_and_output_views():
    """q and out as views with padded token and head strides."""
    sa = _sa()
    case = workloads.make_decode([400, 90], 512, 4, seed=811, poison=True, q_len=4)
    q_buf = torch.zeros((2, 4, 64, 128), dtype=torch.bfloat16)
    q_buf[..., :64] = case.q
    q_view = q_buf.cuda()[..., :64]
    k, v, sinks, sl = _dev(case.k, case.v, case.sinks, case.seqlens_k)
    ws = sa.decode_workspace(8, 64, 8, 4, "cuda")
    out_buf = torch.zeros((2, 5, 64, 64), dtype=torch.bfloat16, device="cuda")
    out_view = out_buf[:, 1:]
    sa.decode_multi_fused(q_view, k, v, sinks, sl, 4, case.scale, ws, out=out_view)
    po, pm, pd = sa.decode_multi_split(q_view, k, v, sinks, sl, 4, case.scale)
    torch.cuda.synchronize()
    ref, _ = oracle_decode_multi(case)
    check_bf16(out_view, ref, "multi fused strided")
    check_multi_partials(po, pm, pd, case, check_bf16, "multi split strided")
    assert torch.all(out_buf[:, 0] == 0), "row outside the view was written"


def test_decode_multi_fp32_tiny():
    sa = _sa()
    case = workloads.make_decode([37, 2, 0], 48, 3, num_q_heads=8, num_kv_heads=2, dtype=torch.float32,
                                 seed=821, poison=True, q_len=3)
    q, k, v, sinks, sl = _dev(case.q, case.k, case.v, case.sinks, case.seqlens_k)
    po, pm, pd = sa.decode_multi_split(q, k, v, sinks, sl, 3, case.scale)
    out = sa.decode_merge(po, pm, pd, out_dtype=torch.float32)
    ws = sa.decode_workspace(9, 8, 2, 3, "cuda")
    fused = sa.decode_multi_fused(q, k, v, sinks, sl, 3, case.scale, ws)
    torch.cuda.synchronize()
    check_multi_partials(po, pm, pd, case, check_f32, "multi tiny f32")
    ref, _ = oracle_decode_multi(case)
    check_f32(out.view(3, 3, 8, 64), ref, "multi tiny f32")
    check_f32(fused, ref, "multi fused tiny f32")


def test_full_multi_decode_8x8192_t4():
    """The decode workload's shape (8 sequences, 8192-key cache, 64/8 heads) with 4 new tokens each;
    every output compared."""
    sa = _sa()
    lens = [8192] * 8
    case = workloads.make_decode(lens, 8192, 8, seed=831, q_len=4)
    q, k, v, sinks, sl = _dev(case.q, case.k, case.v, case.sinks, case.seqlens_k)
    ws = sa.decode_workspace(32, 64, 8, 8, "cuda")
    out = sa.decode_multi_fused(q, k, v, sinks, sl, 8, case.scale, ws)
    torch.cuda.synchronize()
    ref, _ = oracle_decode_multi(case)
    check_bf16(out, ref, "multi full t4")


def test_graph_replays_multi_token_decode_moe_and_linear():
    """Replays of one graph holding the multi-token fused decode (its counters must be left zero by
    each replay), the MoE routing and both linear layers equal their eager results every time."""
    sa = _sa()
    dec = workloads.make_decode([700, 33, 1024, 5] * 16, 1024, 8, seed=51, q_len=4)
    q, k, v, s, sl = _dev(dec.q, dec.k, dec.v, dec.sinks, dec.seqlens_k)
    ws = sa.decode_workspace(64 * 4, 64, 8, 8, "cuda")
    out = torch.empty((64, 4, 64, 64), dtype=torch.bfloat16, device="cuda")
    g = torch.Generator().manual_seed(52)
    logits = torch.randn((4096, 128), generator=g).to(torch.bfloat16).cuda()
    ids = torch.empty((4096, 4), dtype=torch.int32, device="cuda")
    wts = torch.empty((4096, 4), dtype=torch.bfloat16, device="cuda")
    x = torch.randn((256, 512), generator=g).to(torch.bfloat16).cuda()
    w = torch.randn((384, 512), generator=g).to(torch.bfloat16).cuda()
    b = torch.randn(384, generator=g).cuda()
    y = torch.empty((256, 384), dtype=torch.bfloat16, device="cuda")
    qx = (torch.randn((256, 512), generator=g) * 2).to(torch.float8_e4m3fn).cuda()
    qw = (torch.randn((384, 512), generator=g) * 2).to(torch.float8_e4m3fn).cuda()
    sx = (torch.rand((256, 4), generator=g) + 0.5).cuda()
    sw = (torch.rand((3, 4), generator=g) * 0.1).cuda()
    y8 = torch.empty((256, 384), dtype=torch.bfloat16, device="cuda")

    def work():
        sa.decode_multi_fused(q, k, v, s, sl, 8, dec.scale, ws, out=out)
        sa.moe_topk_softmax(logits, 4, ids=ids, weights=wts)
        sa.linear_bias(x, w, b, out=y)
        sa.linear_fp8_block_scaled(qx, sx, qw, sw, b, out=y8)

    work()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (out, ids, wts, y, y8)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    for rep in range(4):
        for t in (out, ids, wts, y, y8):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, e in zip((out, ids, wts, y, y8), eager):
            assert torch.equal(t, e), f"replay {rep}"
        work()  # eager work between replays
        torch.cuda.synchronize()
    counter_bytes = sa._lib.lib.sinkattn_decode_workspace_counter_bytes(64 * 4, 8)
    assert torch.count_nonzero(ws[:counter_bytes]).item() == 0
