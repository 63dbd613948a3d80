"""Plain float64 CPU oracle for the bias GEMM and the FP8 GEMM with 128 x 128 block scaling.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module. The HIP library never calls it and shares no code with it.

What it computes (source: the blog post "GPT-OSS on Day 0", Perplexity, 2025). The section
"GPT-OSS on Hopper" chooses FP8 with 128x128 block scaling as the quantisation scheme and extends
the DeepGEMM kernels to support a bias term; section "Kernels for GPT-OSS" adds the bias by starting
the matrix-core accumulators at bias values loaded from memory, once per output (MN) block.

Readings taken where the pages are silent (each one is also listed in the design notes):

* The GEMM is a linear layer: Y[m, n] = sum_k X[m, k] W[n, k] + bias[n] (W stored [N, K], as the
  weights of a linear layer are); bias is one value per output column.
* FP8 is the OCP E4M3 format (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities;
  S.1111.111 is NaN; largest finite 448), the FP8 format of the hardware targeted here.
* "128x128 block scaling": one fp32 scale per 128 x 128 block of W ([ceil(N/128), K/128]). The pages
  do not say how the activations are scaled; here X carries one fp32 scale per row and 128-column
  block ([M, K/128]), which includes a 128 x 128 activation block as the case of 128 equal rows.
  A block's contribution is scale_x[m, kb] * scale_w[n // 128, kb] * sum over its 128 k of x * w.
"""
from __future__ import annotations

import numpy as np

BLOCK = 128


def e4m3_to_float(codes) -> np.ndarray:
    """Decode OCP E4M3 bytes to float64 from the format definition (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = sign * (1.0 + man / 8.0) * np.exp2(exp - 7.0)
    subnormal = sign * (man / 8.0) * np.exp2(-6.0)
    out = np.where(exp == 0, subnormal, normal)
    return np.where((exp == 0xF) & (man == 0x7), np.nan, out)


def gemm_bias(x, w, bias=None) -> np.ndarray:
    """Y = X W^T + bias in float64. x [M, K], w [N, K], bias [N] or None."""
    y = np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y


def gemm_fp8_block_scaled(x_codes, scale_x, w_codes, scale_w, bias=None) -> np.ndarray:
    """Block-scaled FP8 GEMM, accumulated block by block as the scheme defines it.

    x_codes [M, K] and w_codes [N, K] are E4M3 bytes, K a multiple of 128; scale_x [M, K/128],
    scale_w [ceil(N/128), K/128]. Each 128-wide k block's exact partial product is scaled by
    scale_x[m, kb] * scale_w[n // 128, kb] and added; the bias starts every output.
    """
    x = e4m3_to_float(x_codes)
    w = e4m3_to_float(w_codes)
    m, k = x.shape
    n = w.shape[0]
    assert k % BLOCK == 0
    sx = np.asarray(scale_x, dtype=np.float64)
    sw = np.asarray(scale_w, dtype=np.float64)
    y = np.zeros((m, n)) if bias is None else np.repeat(np.asarray(bias, dtype=np.float64)[None, :], m, axis=0)
    col_block = np.arange(n) // BLOCK
    for kb in range(k // BLOCK):
        ks = slice(kb * BLOCK, (kb + 1) * BLOCK)
        partial = x[:, ks] @ w[:, ks].T
        y += partial * sx[:, kb][:, None] * sw[col_block, kb][None, :]
    return y
