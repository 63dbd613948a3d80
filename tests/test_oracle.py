"""Pins of the CPU oracle against things other than itself (CPU only).

The oracle follows "GPT-OSS on Day 0" (Perplexity), section "Kernels for GPT-OSS" / "Sink
attention".  Each test below fixes one part of it with a closed form, a 50-digit brute force, the
float64 PyTorch SDPA library routine, an identity or an invariance, chosen so that a plausible
slip (a dropped sink term, the sink in every chunk, a wrong head mapping, a transposed operand, a
missing scale, a wrong causal offset) fails at least one of them.  The "mutation" tests plant such
slips in the oracle's own building blocks and check that the pins catch them.
"""
from __future__ import annotations

import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.txt")
D = 64


# ----------------------------------------------------------------------------- helpers
def _logit(tok: str) -> float:
    tok = tok.strip()
    if tok == "-inf":
        return float("-inf")
    assert tok.startswith("ln:"), tok
    return math.log(Fraction(tok[3:]))


def _list(field: str):
    field = field.strip()
    return [] if not field else [t for t in field.split(",")]


def _golden_rows():
    plain, chunked = [], []
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.rstrip("\n")
            if not line.strip() or line.lstrip().startswith("#"):
                continue
            parts = [p.strip() for p in line.split("|")]
            if parts[0].startswith("CHUNKED "):
                chunked.append(parts)
            else:
                plain.append(parts)
    return plain, chunked


def _exact_logit_inputs(logits):
    """q, k with scale 1/8 whose scaled scores equal ``logits`` exactly; v one-hot per key."""
    n = len(logits)
    q = np.zeros(D)
    q[0] = 8.0
    k = np.zeros((n, D))
    k[:, 0] = logits
    v = np.zeros((n, D))
    for j in range(n):
        v[j, j] = 1.0
    return q, k, v


def _sdpa(q, k, v, scale, causal=False, mask=None):
    """float64 CPU scaled_dot_product_attention on [B, H, L, D] tensors."""
    return F.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=None if mask is None else torch.from_numpy(mask), is_causal=causal,
        scale=scale).numpy()


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------------------------- golden
PLAIN, CHUNKED = _golden_rows()


@pytest.mark.parametrize("row", PLAIN, ids=[r[0] for r in PLAIN])
def test_golden_closed_forms(row):
    name, logits_f, sink_f, w_f, ws_f, lse_f = row
    logits = [_logit(t) for t in _list(logits_f)]
    sink = _logit(sink_f)
    weights = [float(Fraction(t)) for t in _list(w_f)]
    q, k, v = _exact_logit_inputs(logits)
    out, lse = oracle.attend(q[None], k, v, sink, 0.125)
    expect_row = np.zeros(D)
    expect_row[:len(weights)] = weights
    np.testing.assert_allclose(out[0], expect_row, rtol=1e-14, atol=1e-15)
    expect_lse = _logit(lse_f)
    if math.isinf(expect_lse):
        assert lse[0] == expect_lse
    else:
        assert lse[0] == pytest.approx(expect_lse, rel=1e-14, abs=1e-14)
    _, p_sink, _ = oracle.sink_softmax(np.array(logits)[None] if logits else np.zeros((1, 0)), sink)
    assert p_sink[0] == pytest.approx(float(Fraction(ws_f)), rel=1e-14, abs=1e-16)


@pytest.mark.parametrize("row", CHUNKED, ids=[r[0] for r in CHUNKED])
def test_golden_chunk_states(row):
    name, logits_f, sink_f, cs_f, m_f, d_f, lse_f = row
    logits = [_logit(t) for t in _list(logits_f)]
    sink = _logit(sink_f)
    cs = int(cs_f)
    m_exp = [_logit(t) for t in _list(m_f)]
    d_exp = [float(Fraction(t)) for t in _list(d_f)]
    chunks = len(m_exp)
    n = len(logits)
    q, k, v = _exact_logit_inputs(logits) if n else (np.eye(1, D)[0] * 8.0, np.zeros((0, D)), np.zeros((0, D)))
    cap = cs * chunks
    kc = np.zeros((1, cap, 1, D))
    vc = np.zeros((1, cap, 1, D))
    kc[0, :n, 0] = k
    vc[0, :n, 0] = v
    po, pm, pd = oracle.decode_split(q[None, None], kc, vc, [sink], [n], chunks, 0.125)
    for c in range(chunks):
        if math.isinf(m_exp[c]):
            assert pm[0, 0, c] == m_exp[c]
        else:
            assert pm[0, 0, c] == pytest.approx(m_exp[c], rel=1e-14, abs=1e-14)
        assert pd[0, 0, c] == pytest.approx(d_exp[c], rel=1e-14, abs=0)
    _, lse = oracle.merge(po, pm, pd)
    assert lse[0, 0] == pytest.approx(_logit(lse_f), rel=1e-14)


# ----------------------------------------------------------------------------- P1: sink = -inf
@pytest.mark.parametrize("causal", [True, False])
def test_p1_no_sink_is_standard_attention(causal):
    rng_q = _rand((1, 8, 37, D), 1)
    rng_k = _rand((1, 2, 37, D), 2)
    rng_v = _rand((1, 2, 37, D), 3)
    scale = 0.125
    # torch's own grouped-query mapping (enable_gqa) is the library reference for the head map
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(rng_q), torch.from_numpy(rng_k), torch.from_numpy(rng_v),
        is_causal=causal, scale=scale, enable_gqa=True).numpy()
    q = rng_q[0].transpose(1, 0, 2)  # [L, H, D]
    k = rng_k[0].transpose(1, 0, 2)
    v = rng_v[0].transpose(1, 0, 2)
    out, _ = oracle.prefill(q, k, v, [-np.inf] * 8, [0, 37], [0, 37], scale, causal)
    np.testing.assert_allclose(out.transpose(1, 0, 2)[None], ref, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------- P2: one key
@pytest.mark.parametrize("s,sink", [(0.3, -1.2), (2.0, 2.0), (-5.0, 4.0), (30.0, -30.0)])
def test_p2_one_key_closed_form(s, sink):
    v = _rand(D, 7)
    q, k, _ = _exact_logit_inputs([s])
    out, lse = oracle.attend(q[None], k, v[None], sink, 0.125)
    sigma = 1.0 / (1.0 + math.exp(sink - s))
    np.testing.assert_allclose(out[0], v * sigma, rtol=1e-14, atol=1e-16)
    assert lse[0] == pytest.approx(math.log(math.exp(s) + math.exp(sink)), rel=1e-14)


# ----------------------------------------------------------------------------- P3: mass
def test_p3_weights_and_sink_sum_to_one():
    z = _rand((50, 33), 11) * 5
    z[:, ::7] = -np.inf
    sink = _rand(50, 12) * 3
    p, ps, lse = oracle.sink_softmax(z, sink)
    np.testing.assert_allclose(p.sum(-1) + ps, 1.0, rtol=0, atol=1e-13)
    assert np.all(p >= 0) and np.all(ps > 0)
    assert np.all(p[:, ::7] == 0)


# ----------------------------------------------------------------------------- P4: split = unsplit
@pytest.mark.parametrize("length", [1, 5, 13])
def test_p4_split_merge_equals_unsplit_all_chunkings(length):
    cap = 16
    q = _rand((2, 4, D), 21)
    k = _rand((2, cap, 2, D), 22)
    v = _rand((2, cap, 2, D), 23)
    sinks = _rand(4, 24) * 2
    lens = [length, max(0, length - 3)]
    ref, ref_lse = oracle.decode(q, k, v, sinks, lens, 0.125)
    for chunks in range(1, cap + 1):
        po, pm, pd = oracle.decode_split(q, k, v, sinks, lens, chunks, 0.125)
        out, lse = oracle.merge(po, pm, pd)
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-13)


def test_p4_mutation_sink_in_every_chunk_is_caught():
    """Planting the sink in every chunk (ignoring the first-chunk rule) must break P4."""
    rng = np.random.default_rng(5)
    z = rng.standard_normal(12)
    vals = rng.standard_normal((12, D))
    sink = 0.7
    ref = oracle.attend(np.eye(1, D) * 8, np.c_[z, np.zeros((12, D - 1))], vals, sink, 0.125)[0][0]
    states = [oracle.chunk_state(z[i:i + 4], vals[i:i + 4], sink) for i in range(0, 12, 4)]
    out_bad, _ = oracle.merge(np.array([s[2] for s in states]), np.array([s[0] for s in states]),
                              np.array([s[1] for s in states]))
    assert np.max(np.abs(out_bad - ref)) > 1e-3
    good = [oracle.chunk_state(z[i:i + 4], vals[i:i + 4], sink if i == 0 else None)
            for i in range(0, 12, 4)]
    out_ok, _ = oracle.merge(np.array([s[2] for s in good]), np.array([s[0] for s in good]),
                             np.array([s[1] for s in good]))
    np.testing.assert_allclose(out_ok, ref, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------- P5: brute force
def _decimal_attention(q, keys, values, sink, scale):
    """50-digit sum_j e^(s_j) v_j / (e^sink + sum_j e^(s_j)) without max subtraction."""
    getcontext().prec = 50
    sc = Decimal(scale)
    ex = []
    for kr in keys:
        s = sc * sum((Decimal(float(a)) * Decimal(float(b)) for a, b in zip(q, kr)), Decimal(0))
        ex.append(s.exp())
    den = sum(ex, Decimal(0)) + (Decimal(0) if math.isinf(sink) else Decimal(sink).exp())
    out = []
    for d in range(len(values[0]) if len(values) else 0):
        num = sum((e * Decimal(float(values[j][d])) for j, e in enumerate(ex)), Decimal(0))
        out.append(float(num / den))
    return np.array(out)


@pytest.mark.parametrize("seed,n,sink", [(1, 1, 0.5), (2, 7, -3.0), (3, 20, 2.5), (4, 9, float("-inf"))])
def test_p5_brute_force_50_digits(seed, n, sink):
    dim = 8
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(dim) * 2
    keys = rng.standard_normal((n, dim))
    vals = rng.standard_normal((n, dim))
    ref = _decimal_attention(q, keys, vals, sink, 0.3)
    out, _ = oracle.attend(q[None], keys, vals, sink, 0.3)
    np.testing.assert_allclose(out[0], ref, rtol=1e-13, atol=1e-15)


# ----------------------------------------------------------------------------- P6: virtual key
def test_p6_sink_is_a_zero_key_with_the_sink_as_its_mask_value():
    """Sink attention = SDPA over [K; 0] and [V; 0] with additive mask [causal | sink_h]."""
    lq = lk = 19
    h_q = 4
    q = _rand((lq, h_q, D), 31)
    k = _rand((lk, h_q, D), 32)
    v = _rand((lk, h_q, D), 33)
    sinks = _rand(h_q, 34) * 2
    out, _ = oracle.prefill(q, k, v, sinks, [0, lq], [0, lk], 0.125, causal=True)
    k_aug = np.concatenate([k, np.zeros((1, h_q, D))], axis=0)
    v_aug = np.concatenate([v, np.zeros((1, h_q, D))], axis=0)
    causal = np.where(np.tril(np.ones((lq, lk), bool)), 0.0, -np.inf)
    mask = np.zeros((1, h_q, lq, lk + 1))
    mask[..., :lk] = causal
    mask[..., lk] = sinks[None, :, None]
    ref = _sdpa(q.transpose(1, 0, 2)[None].copy(), k_aug.transpose(1, 0, 2)[None].copy(),
                v_aug.transpose(1, 0, 2)[None].copy(), 0.125, mask=mask)
    np.testing.assert_allclose(out, ref[0].transpose(1, 0, 2), rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------- P7: decode = prefill
def test_p7_decode_of_last_row_equals_prefill_last_row():
    n = 23
    q = _rand((n, 8, D), 41)
    k = _rand((n, 2, D), 42)
    v = _rand((n, 2, D), 43)
    sinks = _rand(8, 44)
    pre, pre_lse = oracle.prefill(q, k, v, sinks, [0, n], [0, n], 0.125, causal=True)
    dec, dec_lse = oracle.decode(q[n - 1][None], k[None], v[None], sinks, [n], 0.125)
    np.testing.assert_allclose(dec[0], pre[n - 1], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dec_lse[0], pre_lse[n - 1], rtol=1e-13)


# ----------------------------------------------------------------------------- P8: GQA mapping
def test_p8_gqa_equals_mha_with_repeated_kv():
    n, h_q, h_kv = 17, 8, 2
    q = _rand((n, h_q, D), 51)
    k = _rand((n, h_kv, D), 52)
    v = _rand((n, h_kv, D), 53)
    sinks = _rand(h_q, 54)
    gqa, _ = oracle.prefill(q, k, v, sinks, [0, n], [0, n], 0.125, True)
    mha, _ = oracle.prefill(q, np.repeat(k, h_q // h_kv, axis=1), np.repeat(v, h_q // h_kv, axis=1),
                            sinks, [0, n], [0, n], 0.125, True)
    np.testing.assert_allclose(gqa, mha, rtol=1e-14, atol=1e-15)
    # a transposed group map (h % Hkv instead of h // G) gives a different answer
    alt, _ = oracle.prefill(q, np.tile(k, (1, h_q // h_kv, 1)), np.tile(v, (1, h_q // h_kv, 1)),
                            sinks, [0, n], [0, n], 0.125, True)
    assert np.max(np.abs(alt - gqa)) > 1e-3


# ----------------------------------------------------------------------------- P9: limits
def test_p9_strong_sink_sends_output_to_zero_and_shift_invariance():
    z = _rand((3, 40), 61) * 2
    vals = _rand((40, D), 62)
    for big in (50.0, 200.0, 700.0):
        p, ps, _ = oracle.sink_softmax(z, big)
        assert np.max(np.abs(p @ vals)) < 40 * math.exp(np.max(z) - big) * np.max(np.abs(vals)) + 1e-300
        assert np.all(ps > 1 - 1e-15)
    p1, ps1, l1 = oracle.sink_softmax(z, 0.4)
    for c in (-300.0, 17.5, 600.0):
        p2, ps2, l2 = oracle.sink_softmax(z + c, 0.4 + c)
        np.testing.assert_allclose(p2, p1, rtol=1e-12, atol=1e-300)
        np.testing.assert_allclose(ps2, ps1, rtol=1e-12)
        np.testing.assert_allclose(l2, l1 + c, rtol=1e-12)


def test_p9_sink_is_not_scaled():
    """Halving the scale changes the key logits but not the sink logit."""
    q, k, _ = _exact_logit_inputs([math.log(3.0)])
    v = np.eye(1, D)
    out, _ = oracle.attend(q[None], k, v, 0.0, 0.0625)  # scaled logit = ln(3)/2
    w = math.sqrt(3.0) / (math.sqrt(3.0) + 1.0)
    assert out[0, 0] == pytest.approx(w, rel=1e-14)


# ----------------------------------------------------------------------------- P10: key order
@pytest.mark.parametrize("causal", [True, False])
def test_p4_prefill_split_merge_equals_unsplit(causal):
    """Split-KV prefill (sink in split 0 only), merged, equals the unsplit prefill for every split
    count, with varlen sequences, an empty sequence, Lq < Lk (append) and splits past the end."""
    lens_q, lens_k = [9, 0, 5, 12], [9, 0, 70, 12]
    cu_q, cu_k = np.cumsum([0] + lens_q), np.cumsum([0] + lens_k)
    q = _rand((cu_q[-1], 4, D), 91)
    k = _rand((cu_k[-1], 2, D), 92)
    v = _rand((cu_k[-1], 2, D), 93)
    sinks = _rand(4, 94) * 2
    ref, ref_lse = oracle.prefill(q, k, v, sinks, cu_q, cu_k, 0.125, causal)
    for splits in range(1, 7):
        for align in (1, 4, 64):
            po, pm, pd = oracle.prefill_split(q, k, v, sinks, cu_q, cu_k, 0.125, causal, splits, align)
            out, lse = oracle.merge(po, pm, pd)
            np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-13)


def test_prefill_split_states_follow_the_chunk_definition_and_boundaries():
    """Each split's state is the chunk state of the row's visible keys inside the split's
    boundaries [j*ks, (j+1)*ks), ks = ceil(Lk / S) rounded up to the alignment."""
    n_q, n_k, splits, align = 6, 23, 3, 4
    q = _rand((n_q, 1, D), 95)
    k = _rand((n_k, 1, D), 96)
    v = _rand((n_k, 1, D), 97)
    sink = 0.3
    assert oracle.split_size(23, 3, 4) == 8 and oracle.split_size(23, 3, 64) == 64
    assert oracle.split_size(128, 2, 64) == 64 and oracle.split_size(129, 2, 64) == 128
    po, pm, pd = oracle.prefill_split(q, k, v, [sink], [0, n_q], [0, n_k], 0.5, True, splits, align)
    for i in range(n_q):
        last = i + n_k - n_q  # bottom-right causal: keys 0..last are visible
        for j in range(splits):
            lo, hi = 8 * j, min(8 * j + 8, last + 1)
            z = 0.5 * np.array([float(q[i, 0] @ k[t, 0]) for t in range(lo, max(lo, hi))])
            m, d, o = oracle.chunk_state(z, v[lo:max(lo, hi), 0], sink if j == 0 else None)
            assert pm[i, 0, j] == pytest.approx(m, abs=0) if math.isinf(m) else pm[i, 0, j] == pytest.approx(m, rel=1e-13)
            assert pd[i, 0, j] == pytest.approx(d, rel=1e-13, abs=0)
            np.testing.assert_allclose(po[i, 0, j], o, rtol=1e-12, atol=1e-14)


def test_prefill_split_mutation_sink_in_every_split_is_caught():
    """The first-chunk rule matters for prefill too: a sink folded into every split breaks the
    merge identity."""
    n = 40
    q = _rand((n, 1, D), 98)
    k = _rand((n, 1, D), 99)
    v = _rand((n, 1, D), 100)
    sink = 1.5
    ref, _ = oracle.prefill(q, k, v, [sink], [0, n], [0, n], 0.125, True)
    po, pm, pd = oracle.prefill_split(q, k, v, [sink], [0, n], [0, n], 0.125, True, 4, 4)
    # Plant the sink in splits 1..3 of every row by refolding its term into (m, d, o).
    for j in range(1, 4):
        m_old, d_old, o_old = pm[:, 0, j], pd[:, 0, j], po[:, 0, j]
        m_new = np.maximum(m_old, sink)
        d_new = np.where(np.isneginf(m_old), 0.0, d_old * np.exp(m_old - m_new)) + np.exp(sink - m_new)
        w_old = np.where(np.isneginf(m_old), 0.0, d_old * np.exp(m_old - m_new))
        po[:, 0, j] = (w_old[:, None] * o_old) / d_new[:, None]
        pm[:, 0, j], pd[:, 0, j] = m_new, d_new
    bad, _ = oracle.merge(po, pm, pd)
    assert np.max(np.abs(bad - ref)) > 1e-3


def test_p10_noncausal_output_is_invariant_under_key_permutation():
    n = 29
    q = _rand((11, 4, D), 71)
    k = _rand((n, 1, D), 72)
    v = _rand((n, 1, D), 73)
    sinks = _rand(4, 74)
    perm = np.random.default_rng(75).permutation(n)
    a, _ = oracle.prefill(q, k, v, sinks, [0, 11], [0, n], 0.125, causal=False)
    b, _ = oracle.prefill(q, k[perm], v[perm], sinks, [0, 11], [0, n], 0.125, causal=False)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)


# ----------------------------------------------------------------------------- the page's online form
def test_online_recurrence_with_sink_init_equals_definition():
    """m started at the sink and d at 1, tile by tile, equals the plain definition."""
    rng = np.random.default_rng(81)
    z = rng.standard_normal(50) * 3
    vals = rng.standard_normal((50, D))
    for sink in (-4.0, 0.0, 1.5, 9.0, float("-inf")):
        ref_p, _, _ = oracle.sink_softmax(z[None], sink)
        ref = ref_p[0] @ vals
        for tile in (1, 7, 16, 50):
            tiles = [z[i:i + tile] for i in range(0, 50, tile)]
            vt = [vals[i:i + tile] for i in range(0, 50, tile)]
            out, m, d = oracle.online_row(tiles, vt, sink)
            np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
            assert m == max(sink, z.max())


def test_online_mutation_dropping_the_sink_term_is_caught():
    """d started at 0 with m at the sink loses the sink's e^0 = 1 and fails the one-key closed form."""
    s, sink = 0.3, 0.1
    v = np.ones((1, D))
    out, _, _ = oracle.online_row([np.array([s])], [v], sink, initial_scale=0.0)
    sigma = 1.0 / (1.0 + math.exp(sink - s))
    assert abs(out[0] - sigma) > 0.1


# ----------------------------------------------------------------------------- causal offset
def test_bottom_right_causal_alignment_for_shorter_query_block():
    """With Lq < Lk, the last query row sees every key, and equals decode of that row."""
    lq, lk = 5, 12
    q = _rand((lq, 2, D), 91)
    k = _rand((lk, 1, D), 92)
    v = _rand((lk, 1, D), 93)
    sinks = _rand(2, 94)
    out, _ = oracle.prefill(q, k, v, sinks, [0, lq], [0, lk], 0.125, causal=True)
    for i in range(lq):
        seen = lk - lq + i + 1
        dec, _ = oracle.decode(q[i][None], k[None], v[None], sinks, [seen], 0.125)
        np.testing.assert_allclose(out[i], dec[0], rtol=1e-13, atol=1e-15)


def test_prefill_at_matches_full_prefill_on_varlen():
    lens = [3, 1, 9, 6]
    cu = np.concatenate([[0], np.cumsum(lens)])
    t = int(cu[-1])
    q = _rand((t, 4, D), 101)
    k = _rand((t, 2, D), 102)
    v = _rand((t, 2, D), 103)
    sinks = _rand(4, 104)
    full, full_lse = oracle.prefill(q, k, v, sinks, cu, cu, 0.125, True)
    tokens = np.repeat(np.arange(t), 4)
    heads = np.tile(np.arange(4), t)
    part, part_lse = oracle.prefill_at(q, k, v, sinks, cu, cu, 0.125, True, tokens, heads)
    np.testing.assert_allclose(part, full[tokens, heads], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(part_lse, full_lse[tokens, heads], rtol=1e-12)


def test_varlen_sequences_do_not_see_each_other():
    """Each packed sequence equals the same sequence run alone."""
    lens = [4, 7, 2]
    cu = np.concatenate([[0], np.cumsum(lens)])
    t = int(cu[-1])
    q = _rand((t, 2, D), 111)
    k = _rand((t, 1, D), 112)
    v = _rand((t, 1, D), 113)
    sinks = _rand(2, 114)
    packed, _ = oracle.prefill(q, k, v, sinks, cu, cu, 0.125, True)
    for b in range(3):
        a, z = cu[b], cu[b + 1]
        alone, _ = oracle.prefill(q[a:z], k[a:z], v[a:z], sinks, [0, z - a], [0, z - a], 0.125, True)
        np.testing.assert_allclose(packed[a:z], alone, rtol=1e-14, atol=1e-16)


# ----------------------------------------------------------------------------- properties
@settings(max_examples=40, deadline=None)
@given(st.integers(0, 12), st.integers(1, 6), st.integers(1, 3), st.floats(-6, 6),
       st.integers(0, 10_000))
def test_property_split_merge_matches_decode(length, chunks, group, sink, seed):
    cap = 12
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, group, D))
    k = rng.standard_normal((1, cap, 1, D)) * 2
    v = rng.standard_normal((1, cap, 1, D))
    ref, ref_lse = oracle.decode(q, k, v, [sink] * group, [length], 0.125)
    po, pm, pd = oracle.decode_split(q, k, v, [sink] * group, [length], chunks, 0.125)
    out, lse = oracle.merge(po, pm, pd)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-11, atol=1e-13)
    # brute force on the unsplit value
    bf = _decimal_attention(q[0, 0], k[0, :length, 0], v[0, :length, 0], sink, 0.125) if length \
        else np.zeros(D)
    np.testing.assert_allclose(ref[0, 0], bf, rtol=1e-12, atol=1e-14)


def test_zero_length_and_dead_rows_are_zero():
    q = _rand((1, 2, D), 121)
    k = np.zeros((1, 4, 1, D))
    out, lse = oracle.decode(q, k, k, [1.0, float("-inf")], [0], 0.125)
    assert np.all(out == 0)
    assert lse[0, 0] == 1.0 and lse[0, 1] == float("-inf")


# ----------------------------------------------------------------------------- multi-token decode
def _multi_case(batch, q_len, cap, lens, h_q, h_kv, seed):
    q = _rand((batch, q_len, h_q, D), seed)
    k = _rand((batch, cap, h_kv, D), seed + 1)
    v = _rand((batch, cap, h_kv, D), seed + 2)
    sinks = _rand(h_q, seed + 3) * 2
    return q, k, v, sinks, np.asarray(lens, dtype=np.int32)


def test_decode_multi_is_sdpa_with_a_sink_key_and_bottom_right_mask():
    """Each sequence: SDPA (float64 library routine) over [K; 0], [V; 0] with additive mask
    [bottom-right causal | sink_h], the KV heads repeated over their query-head groups."""
    q, k, v, sinks, lens = _multi_case(3, 5, 21, [21, 9, 6], 8, 2, 700)
    out, lse = oracle.decode_multi(q, k, v, sinks, lens, 0.125)
    for b, n in enumerate(lens):
        kb = np.repeat(k[b, :n], 4, axis=1)  # [n, Hq, D]
        vb = np.repeat(v[b, :n], 4, axis=1)
        k_aug = np.concatenate([kb, np.zeros((1, 8, D))], axis=0).transpose(1, 0, 2)[None].copy()
        v_aug = np.concatenate([vb, np.zeros((1, 8, D))], axis=0).transpose(1, 0, 2)[None].copy()
        mask = np.zeros((1, 8, 5, n + 1))
        for t in range(5):
            mask[0, :, t, n - 5 + t + 1:n] = -np.inf  # token t sees keys j <= n - 5 + t
        mask[..., n] = sinks[None, :, None]
        ref = _sdpa(q[b].transpose(1, 0, 2)[None].copy(), k_aug, v_aug, 0.125, mask=mask)
        np.testing.assert_allclose(out[b], ref[0].transpose(1, 0, 2), rtol=1e-12, atol=1e-13)
    assert np.all(np.isfinite(lse))


def test_decode_multi_rows_equal_prefill_of_the_last_rows():
    """Token t of a sequence of L keys is prefill row t of Lq = T queries against Lk = L keys."""
    q, k, v, sinks, lens = _multi_case(2, 4, 30, [30, 11], 4, 4, 710)
    out, lse = oracle.decode_multi(q, k, v, sinks, lens, 0.2)
    for b, n in enumerate(lens):
        pre, pre_lse = oracle.prefill(q[b], k[b, :n], v[b, :n], sinks, [0, 4], [0, n], 0.2, causal=True)
        np.testing.assert_allclose(out[b], pre, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(lse[b], pre_lse, rtol=1e-13)


def test_decode_multi_with_one_token_is_decode():
    q, k, v, sinks, lens = _multi_case(3, 1, 17, [17, 4, 0], 8, 2, 720)
    out, lse = oracle.decode_multi(q, k, v, sinks, lens, 0.125)
    ref, ref_lse = oracle.decode(q[:, 0], k, v, sinks, lens, 0.125)
    np.testing.assert_allclose(out[:, 0], ref, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse[:, 0], ref_lse, rtol=1e-14)
    po, pm, pd = oracle.decode_multi_split(q, k, v, sinks, lens, 3, 0.125)
    so, sm, sd = oracle.decode_split(q[:, 0], k, v, sinks, lens, 3, 0.125)
    np.testing.assert_array_equal(po, so)
    np.testing.assert_array_equal(pm, sm)
    np.testing.assert_array_equal(pd, sd)


def test_decode_multi_rows_without_keys_put_all_weight_on_the_sink():
    """With fewer keys than tokens, token t sees L - T + 1 + t <= 0 keys: out = 0, lse = sink."""
    q, k, v, sinks, lens = _multi_case(1, 6, 8, [3], 2, 1, 730)
    out, lse = oracle.decode_multi(q, k, v, sinks, lens, 0.125)
    for t in range(3):  # 3 - 6 + 1 + t <= 0 for t <= 2
        np.testing.assert_array_equal(out[0, t], np.zeros((2, D)))
        np.testing.assert_allclose(lse[0, t], sinks, rtol=1e-15)
    assert np.all(np.abs(out[0, 3:]) > 0)


@pytest.mark.parametrize("chunks", [1, 2, 3, 5, 8, 40])
def test_decode_multi_split_merge_equals_unsplit(chunks):
    """Chunk borders fall inside the masked last T - 1 keys for some chunkings; lengths below T
    leave rows with no keys."""
    q, k, v, sinks, lens = _multi_case(4, 5, 40, [40, 23, 5, 2], 8, 4, 740)
    ref, ref_lse = oracle.decode_multi(q, k, v, sinks, lens, 0.125)
    po, pm, pd = oracle.decode_multi_split(q, k, v, sinks, lens, chunks, 0.125)
    out, lse = oracle.merge(po, pm, pd)
    np.testing.assert_allclose(out.reshape(ref.shape), ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse.reshape(ref_lse.shape), ref_lse, rtol=1e-12)


def test_decode_multi_split_mutation_sink_in_every_chunk_is_caught():
    q, k, v, sinks, lens = _multi_case(1, 3, 24, [24], 2, 1, 750)
    ref, _ = oracle.decode_multi(q, k, v, sinks, lens, 0.125)
    po, pm, pd = oracle.decode_multi_split(q, k, v, sinks, lens, 4, 0.125)
    cs = oracle.chunk_size(24, 4)
    for t in range(3):
        seen = 24 - 3 + 1 + t
        for h in range(2):
            for c in range(1, 4):
                lo, hi = c * cs, min((c + 1) * cs, seen)
                z = 0.125 * (k[0, lo:hi, 0] @ q[0, t, h])
                m, d, o = oracle.chunk_state(z, v[0, lo:hi, 0], sinks[h])
                po[t, h, c], pm[t, h, c], pd[t, h, c] = o, m, d
    out, _ = oracle.merge(po, pm, pd)
    assert np.max(np.abs(out.reshape(ref.shape) - ref)) > 1e-3
