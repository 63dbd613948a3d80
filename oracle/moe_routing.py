"""Plain float64 CPU oracle for the MoE routing softmax taken after the top-K expert choice.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module. The HIP library never calls it and shares no code with it.

What it computes (source: the blog post "GPT-OSS on Day 0", Perplexity, 2025; the model outline in
"GPT-OSS on Hopper" lists a softmax after the top-K choice for the expert weights, and section
"Kernels for GPT-OSS" says the routing scores were changed so the softmax runs over the top-K chosen
experts only, where DeepSeek-style models take it over all experts, and that computing the expert
weights in bfloat16 was essential for accuracy).

Readings taken where the pages are silent (each one is also listed in the design notes):

* Inputs are the router logits of each token, one per expert ([T, E]); the router GEMM that makes
  them is not part of this step. The pages give neither E nor K: both are parameters.
* The top-K experts are the K largest logits, compared exactly as stored; among equal logits the
  lower expert index comes first. Returned ids are ordered by (logit descending, index ascending).
* "Expert weights in bfloat16": the softmax over the K chosen logits is exact arithmetic here
  (float64); the library computes it in float32 and rounds the weights to bf16, which is what a
  bf16 softmax produces (float32 internally, bf16 result). Tests compare within one bf16 ulp.
* The contrast the page draws (softmax over all experts, then the top-K of it) is the
  ``over_all=True`` mode: the same ids, weights normalised over all E experts.
* A token whose largest logit is -inf has no finite weight: its weights are defined as 0.
"""
from __future__ import annotations

import numpy as np


def topk_experts(logits, k: int) -> np.ndarray:
    """Ids [T, K] of the K largest logits per row, ordered by (logit descending, index ascending)."""
    logits = np.asarray(logits, dtype=np.float64)
    t, e = logits.shape
    assert 1 <= k <= e
    ids = np.zeros((t, k), dtype=np.int64)
    for row in range(t):
        order = sorted(range(e), key=lambda j: (-logits[row, j], j))
        ids[row] = order[:k]
    return ids


def moe_topk_softmax(logits, k: int, over_all: bool = False):
    """Routing weights of the top-K experts: ``(ids [T, K] int64, weights [T, K] float64)``.

    ``over_all=False`` (GPT-OSS): softmax over the K chosen logits only, so each row sums to 1.
    ``over_all=True`` (the DeepSeek-style contrast): softmax over all E logits, weights of the K.
    """
    logits = np.asarray(logits, dtype=np.float64)
    ids = topk_experts(logits, k)
    chosen = np.take_along_axis(logits, ids, axis=1)
    pool = logits if over_all else chosen
    top = chosen[:, :1]  # the largest logit of the row (ids are ordered)
    weights = np.zeros(chosen.shape)
    live = np.isfinite(top[:, 0])
    e_chosen = np.exp(chosen[live] - top[live])
    e_pool = np.exp(pool[live] - top[live])
    weights[live] = e_chosen / e_pool.sum(axis=1, keepdims=True)
    return ids, weights
