"""Pins of the MoE routing oracle (CPU): closed forms, library routines, invariants, a planted mistake.

Source: "GPT-OSS on Day 0" (Perplexity): softmax after the top-K choice of experts, over the K chosen
experts only ("GPT-OSS on Hopper" outline; "Kernels for GPT-OSS", MoE routing paragraph).
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "moe_topk_closed_forms.txt")


def _logit(tok):
    tok = tok.strip()
    if tok == "-inf":
        return float("-inf")
    assert tok.startswith("ln:"), tok
    return math.log(Fraction(tok[3:]))


def _rows():
    out = []
    with open(GOLDEN) as fh:
        for line in fh:
            if line.strip() and not line.lstrip().startswith("#"):
                out.append([p.strip() for p in line.rstrip("\n").split("|")])
    return out


ROWS = _rows()


@pytest.mark.parametrize("row", ROWS, ids=[r[0] for r in ROWS])
def test_golden_closed_forms(row):
    name, mode, logits_f, k_f, ids_f, w_f = row
    logits = np.array([[_logit(t) for t in logits_f.split(",")]])
    ids, w = oracle.moe_topk_softmax(logits, int(k_f), over_all=(mode == "all"))
    assert ids[0].tolist() == [int(t) for t in ids_f.split(",")]
    np.testing.assert_allclose(w[0], [float(Fraction(t)) for t in w_f.split(",")], rtol=1e-14, atol=0)


def _bf16_logits(t, e, seed, scale=1.0):
    """Random logits with bf16 values (many exact ties among 128 experts)."""
    g = torch.Generator().manual_seed(seed)
    return (torch.randn((t, e), generator=g) * scale).to(torch.bfloat16).double().numpy()


def test_ids_match_a_lexicographic_library_sort():
    """ids = the first K of numpy's lexsort by (-logit, index), row by row; ties are common here."""
    logits = _bf16_logits(64, 128, 11)
    ids = oracle.topk_experts(logits, 6)
    ties = 0
    for r in range(logits.shape[0]):
        order = np.lexsort((np.arange(128), -logits[r]))
        assert ids[r].tolist() == order[:6].tolist()
        ties += len(logits[r]) - len(np.unique(logits[r]))
    assert ties > 100  # the case exercises the tie rule


def test_chosen_set_dominates_the_rest():
    logits = _bf16_logits(32, 32, 12)
    ids = oracle.topk_experts(logits, 4)
    for r in range(32):
        chosen = set(ids[r].tolist())
        rest = [j for j in range(32) if j not in chosen]
        assert min(logits[r, list(chosen)]) >= max(logits[r, rest])
        # an expert left out with the same logit as a chosen one has a higher index
        cut = min(logits[r, list(chosen)])
        assert all(j > max(i for i in chosen if logits[r, i] == cut) for j in rest if logits[r, j] == cut)


def test_k_equals_e_is_the_library_softmax():
    logits = _bf16_logits(16, 32, 13, scale=3.0)
    ids, w = oracle.moe_topk_softmax(logits, 32)
    ref = torch.softmax(torch.from_numpy(logits), dim=-1).numpy()
    np.testing.assert_allclose(w, np.take_along_axis(ref, ids, axis=1), rtol=1e-13, atol=0)


def test_over_all_mode_is_the_library_softmax_at_the_chosen_ids():
    logits = _bf16_logits(16, 128, 14, scale=2.0)
    ids, w = oracle.moe_topk_softmax(logits, 4, over_all=True)
    ref = torch.softmax(torch.from_numpy(logits), dim=-1).numpy()
    np.testing.assert_allclose(w, np.take_along_axis(ref, ids, axis=1), rtol=1e-13, atol=0)


def test_topk_weights_are_the_library_softmax_of_the_chosen_logits_and_sum_to_one():
    logits = _bf16_logits(16, 128, 15, scale=2.0)
    ids, w = oracle.moe_topk_softmax(logits, 4)
    chosen = torch.from_numpy(np.take_along_axis(logits, ids, axis=1))
    np.testing.assert_allclose(w, torch.softmax(chosen, dim=-1).numpy(), rtol=1e-13, atol=0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)  # ordered by logit, so weights do not increase


def test_shift_invariance():
    logits = _bf16_logits(8, 64, 16)
    for over_all in (False, True):
        ids, w = oracle.moe_topk_softmax(logits, 5, over_all)
        ids2, w2 = oracle.moe_topk_softmax(logits + 37.0, 5, over_all)
        assert np.array_equal(ids, ids2)
        np.testing.assert_allclose(w, w2, rtol=1e-12)


def test_mutation_softmax_over_all_experts_is_caught():
    """The planted mistake the page warns about: normalising over all experts instead of the K chosen."""
    logits = _bf16_logits(8, 128, 17)
    _, w = oracle.moe_topk_softmax(logits, 4)
    _, w_all = oracle.moe_topk_softmax(logits, 4, over_all=True)
    np.testing.assert_allclose(w.sum(axis=1), 1.0)
    assert np.max(np.abs(w - w_all)) > 0.05
