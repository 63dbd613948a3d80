"""Seeded synthetic inputs for sink attention, shaped like GPT-OSS attention layers.

This module holds no attention arithmetic: only random draws, tensor shapes and index
bookkeeping (prefix sums of sequence lengths).  Both the HIP path and the CPU oracle are fed from
it; neither is imported here.

Every tensor is drawn on the CPU from ``torch.Generator`` objects seeded from ``1000 + config``
(lengths from that seed; each tensor group from the next seeds), in a fixed order (lengths, q, k,
v, outlier mask, sinks).  Values are drawn in float32 and rounded to
bfloat16 with round-to-nearest-even where the config is bf16, so the GPU and the oracle see the
same bits on every machine.

Workloads (head_dim 64, GPT-OSS grouping of 64 query heads over 8 KV heads):

* 1 ``tiny``: causal prefill, 1 sequence of 128 tokens, 4 query heads over 1 KV head, fp32
  N(0,1) Q/K/V, sinks N(0,1), scale 1/8; decode of one query against the same 128 keys in 4 chunks.
* 2 ``decode``: 8 sequences, every KV length 8192, bf16 N(0,1), sinks U(-2,2), chunk 1024.
* 3 ``prefill``: 1 causal sequence of 8192 tokens, bf16 N(0,1), sinks U(-2,2), scale 1/8.
* 4 ``long_decode``: 32 sequences, KV lengths uniform in [16384, 32768], capacity 32768,
  bf16 N(0,1) with 1% of K rows scaled by 8 (outlier logits), sinks U(-4,4), chunk 2048.
* 5 ``mixed``: decode of 128 sequences with KV lengths uniform in [1, 8192] (capacity 8192,
  8 chunks) plus causal varlen prefill of 16 sequences with lengths uniform in [512, 4096].
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

HEAD_DIM = 64
SCALE = 1.0 / math.sqrt(HEAD_DIM)

NAMES = {1: "tiny", 2: "decode", 3: "prefill", 4: "long_decode", 5: "mixed"}


@dataclass
class PrefillCase:
    """Packed varlen prefill inputs (CPU tensors)."""

    q: torch.Tensor            # [Tq, Hq, D]
    k: torch.Tensor            # [Tk, Hkv, D]
    v: torch.Tensor            # [Tk, Hkv, D]
    sinks: torch.Tensor        # [Hq] float32
    cu_seqlens_q: torch.Tensor  # [B+1] int32
    cu_seqlens_k: torch.Tensor  # [B+1] int32
    scale: float = SCALE
    causal: bool = True

    @property
    def lens_q(self):
        return (self.cu_seqlens_q[1:] - self.cu_seqlens_q[:-1]).tolist()

    @property
    def lens_k(self):
        return (self.cu_seqlens_k[1:] - self.cu_seqlens_k[:-1]).tolist()


@dataclass
class DecodeCase:
    """Decode inputs against a padded KV cache (CPU tensors): one or q_len new tokens per sequence."""

    q: torch.Tensor          # [B, Hq, D], or [B, T, Hq, D] for multi-token decode
    k: torch.Tensor          # [B, Lcap, Hkv, D]
    v: torch.Tensor          # [B, Lcap, Hkv, D]
    sinks: torch.Tensor      # [Hq] float32
    seqlens_k: torch.Tensor  # [B] int32
    num_chunks: int
    scale: float = SCALE


@dataclass
class Workload:
    config: int
    name: str
    prefill: PrefillCase | None = None
    decode: DecodeCase | None = None
    extra: dict = field(default_factory=dict)


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _normal(shape, gen, dtype):
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(dtype)


def _uniform(shape, lo, hi, gen):
    return torch.rand(shape, generator=gen, dtype=torch.float32) * (hi - lo) + lo


def _int_uniform(n, lo, hi, gen):
    """n integers uniform on the closed range [lo, hi]."""
    return torch.randint(lo, hi + 1, (n,), generator=gen, dtype=torch.int64)


def _cu(lens) -> torch.Tensor:
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def make_prefill(lens_q, lens_k=None, *, num_q_heads=64, num_kv_heads=8, head_dim=HEAD_DIM,
                 dtype=torch.bfloat16, sink_range=(-2.0, 2.0), sink_normal=False, seed=0,
                 scale=SCALE, causal=True) -> PrefillCase:
    """Packed varlen prefill batch: q/k/v N(0,1), sinks U(sink_range) (or N(0,1))."""
    lens_k = list(lens_q) if lens_k is None else list(lens_k)
    gen = _gen(seed)
    t_q, t_k = int(sum(lens_q)), int(sum(lens_k))
    q = _normal((t_q, num_q_heads, head_dim), gen, dtype)
    k = _normal((t_k, num_kv_heads, head_dim), gen, dtype)
    v = _normal((t_k, num_kv_heads, head_dim), gen, dtype)
    sinks = (torch.randn(num_q_heads, generator=gen) if sink_normal
             else _uniform(num_q_heads, *sink_range, gen))
    return PrefillCase(q, k, v, sinks.float(), _cu(lens_q), _cu(lens_k), scale, causal)


def make_decode(lens, capacity, num_chunks, *, num_q_heads=64, num_kv_heads=8,
                head_dim=HEAD_DIM, dtype=torch.bfloat16, sink_range=(-2.0, 2.0),
                sink_normal=False, outlier_p=0.0, outlier_scale=8.0, seed=0, scale=SCALE,
                poison=False, q_len=None) -> DecodeCase:
    """KV cache [B, capacity, Hkv, D]; rows at or past each length are zero, or NaN if ``poison``.

    q is [B, Hq, D], or [B, q_len, Hq, D] for multi-token decode (the lengths then count the
    q_len new tokens, whose keys are already in the cache).

    Only the valid rows are drawn (one sequence at a time, to bound host memory).  With
    ``outlier_p`` > 0 each valid K row (b, t, g) is independently multiplied by ``outlier_scale``
    with that probability (8 is a power of two, so the scaling is exact in bf16).
    """
    gen = _gen(seed)
    batch = len(lens)
    fill = float("nan") if poison else 0.0
    q_shape = (batch, num_q_heads, head_dim) if q_len is None else (batch, q_len, num_q_heads, head_dim)
    q = _normal(q_shape, gen, dtype)
    k = torch.full((batch, capacity, num_kv_heads, head_dim), fill, dtype=dtype)
    v = torch.full((batch, capacity, num_kv_heads, head_dim), fill, dtype=dtype)
    for b, n in enumerate(lens):
        k[b, :n] = _normal((int(n), num_kv_heads, head_dim), gen, dtype)
    for b, n in enumerate(lens):
        v[b, :n] = _normal((int(n), num_kv_heads, head_dim), gen, dtype)
    if outlier_p > 0:
        for b, n in enumerate(lens):
            hit = torch.rand((int(n), num_kv_heads), generator=gen) < outlier_p
            rows = k[b, :n]
            rows[hit] = (rows[hit].float() * outlier_scale).to(dtype)
    sinks = (torch.randn(num_q_heads, generator=gen) if sink_normal
             else _uniform(num_q_heads, *sink_range, gen))
    seqlens = torch.tensor([int(n) for n in lens], dtype=torch.int32)
    return DecodeCase(q, k, v, sinks.float(), seqlens, int(num_chunks), scale)


def make(config: int, *, poison=False) -> Workload:
    """The five named workloads; seed = 1000 + config."""
    seed = 1000 + int(config)
    name = NAMES[int(config)]
    if config == 1:
        pre = make_prefill([128], num_q_heads=4, num_kv_heads=1, dtype=torch.float32,
                           sink_normal=True, seed=seed)
        gen = _gen(seed + 100)
        q_fresh = torch.randn((1, 4, HEAD_DIM), generator=gen, dtype=torch.float32)
        k_cache = pre.k.reshape(1, 128, 1, HEAD_DIM).clone()
        v_cache = pre.v.reshape(1, 128, 1, HEAD_DIM).clone()
        dec = DecodeCase(q_fresh, k_cache, v_cache, pre.sinks.clone(),
                         torch.tensor([128], dtype=torch.int32), 4)
        # The same keys queried by the prefill's last row: decode must equal prefill row 127.
        dec_last = DecodeCase(pre.q[127:128].clone(), k_cache, v_cache, pre.sinks.clone(),
                              torch.tensor([128], dtype=torch.int32), 4)
        return Workload(1, name, prefill=pre, decode=dec, extra={"decode_last_row": dec_last})
    if config == 2:
        dec = make_decode([8192] * 8, 8192, 8, seed=seed, poison=poison)
        return Workload(2, name, decode=dec)
    if config == 3:
        return Workload(3, name, prefill=make_prefill([8192], seed=seed))
    if config == 4:
        gen = _gen(seed)
        lens = _int_uniform(32, 16384, 32768, gen).tolist()
        dec = make_decode(lens, 32768, 16, sink_range=(-4.0, 4.0), outlier_p=0.01,
                          seed=seed + 1, poison=poison)
        return Workload(4, name, decode=dec)
    if config == 5:
        gen = _gen(seed)
        dec_lens = _int_uniform(128, 1, 8192, gen).tolist()
        pre_lens = _int_uniform(16, 512, 4096, gen).tolist()
        dec = make_decode(dec_lens, 8192, 8, seed=seed + 1, poison=poison)
        pre = make_prefill(pre_lens, seed=seed + 2)
        return Workload(5, name, prefill=pre, decode=dec)
    raise ValueError(f"unknown workload {config}")


def decode_kv_bytes(case: DecodeCase) -> int:
    """K and V bytes a decode must read: sum of valid lengths x Hkv x D x element size x 2."""
    hkv, dim = case.k.shape[2], case.k.shape[3]
    return int(case.seqlens_k.sum()) * hkv * dim * case.k.element_size() * 2


def prefill_causal_pairs(case: PrefillCase) -> int:
    """Allowed (query, key) pairs per head, summed over sequences (bottom-right causal)."""
    import numpy as np

    total = 0
    for n_q, n_k in zip(case.lens_q, case.lens_k):
        if not case.causal:
            total += n_q * n_k
            continue
        rows = np.arange(n_q, dtype=np.int64)
        total += int(np.clip(rows + (n_k - n_q) + 1, 0, n_k).sum())
    return total
