"""Pins of the GEMM oracle (CPU): E4M3 decoding, brute force, closed forms, the dequantise identity.

Source: "GPT-OSS on Day 0" (Perplexity): FP8 with 128x128 block scaling and a bias term added by
starting the accumulators at the bias ("GPT-OSS on Hopper"; "Kernels for GPT-OSS").
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def test_e4m3_decode_matches_the_library_format_for_all_codes():
    codes = np.arange(256)
    ref = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_to_float(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got)) and nan.sum() == 2
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("code,value", [(0x38, 1.0), (0xB8, -1.0), (0x7E, 448.0), (0x01, 2.0 ** -9),
                                        (0x08, 2.0 ** -6), (0x00, 0.0), (0x3C, 1.5), (0x40, 2.0)])
def test_e4m3_closed_forms(code, value):
    assert oracle.e4m3_to_float([code])[0] == value


def test_gemm_bias_brute_force_exact():
    rng = np.random.default_rng(1)
    x = rng.integers(-5, 6, size=(3, 7))
    w = rng.integers(-5, 6, size=(4, 7))
    b = rng.integers(-9, 10, size=4)
    y = oracle.gemm_bias(x, w, b)
    for m in range(3):
        for n in range(4):
            assert y[m, n] == sum(Fraction(int(x[m, k])) * int(w[n, k]) for k in range(7)) + int(b[n])


def test_gemm_bias_closed_forms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 8))
    b = rng.standard_normal(8)
    np.testing.assert_array_equal(oracle.gemm_bias(x, np.eye(8), b), x + b)
    np.testing.assert_allclose(oracle.gemm_bias(x, np.ones((3, 8)), b[:3]), x.sum(axis=1, keepdims=True) + b[:3],
                               rtol=1e-14)
    np.testing.assert_array_equal(oracle.gemm_bias(np.zeros((2, 8)), np.ones((3, 8)), b[:3]), np.tile(b[:3], (2, 1)))


def _fp8_case(m, n, k, seed):
    rng = np.random.default_rng(seed)
    # finite E4M3 codes only (0x7F / 0xFF are NaN)
    x = rng.integers(0, 256, size=(m, k))
    w = rng.integers(0, 256, size=(n, k))
    x[(x & 0x7F) == 0x7F] = 0x38
    w[(w & 0x7F) == 0x7F] = 0x38
    sx = rng.uniform(0.5, 2.0, size=(m, k // 128))
    sw = rng.uniform(0.5, 2.0, size=(-(-n // 128), k // 128))
    b = rng.standard_normal(n)
    return x, sx, w, sw, b


def test_fp8_block_scaled_equals_gemm_of_dequantised_operands():
    """Distributing the scales: X_deq[m, k] = sx[m, k//128] x[m, k], W_deq[n, k] = sw[n//128, k//128]
    w[n, k]; the block-wise accumulation equals the plain GEMM of the dequantised operands."""
    x, sx, w, sw, b = _fp8_case(40, 300, 384, 3)
    y = oracle.gemm_fp8_block_scaled(x, sx, w, sw, b)
    xd = oracle.e4m3_to_float(x) * np.repeat(sx, 128, axis=1)
    wd = oracle.e4m3_to_float(w) * np.repeat(np.repeat(sw, 128, axis=1), 128, axis=0)[:300]
    ref = xd @ wd.T + b
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-9 * np.abs(ref).max())


def test_fp8_unit_scales_on_small_integers_are_exact():
    """Codes of small integers (E4M3 represents 0..16 exactly), unit scales: the exact integer product."""
    rng = np.random.default_rng(4)
    ints = rng.integers(-8, 9, size=(6, 256))
    intw = rng.integers(-8, 9, size=(5, 256))
    enc = {v: int(torch.tensor([float(v)]).to(torch.float8_e4m3fn).view(torch.uint8)[0]) for v in range(-8, 9)}
    x = np.vectorize(enc.get)(ints)
    w = np.vectorize(enc.get)(intw)
    y = oracle.gemm_fp8_block_scaled(x, np.ones((6, 2)), w, np.ones((1, 2)), None)
    assert np.array_equal(y, (ints @ intw.T).astype(np.float64))


def test_fp8_mutation_wrong_weight_scale_block_is_caught():
    """The planted mistake: indexing the weight scale by k block only (one scale per column block
    ignored) changes the result."""
    x, sx, w, sw, b = _fp8_case(8, 256, 256, 5)
    y = oracle.gemm_fp8_block_scaled(x, sx, w, sw, b)
    sw_wrong = np.repeat(sw[:1], sw.shape[0], axis=0)  # every column block takes block 0's scales
    y_wrong = oracle.gemm_fp8_block_scaled(x, sx, w, sw_wrong, b)
    assert np.max(np.abs(y - y_wrong)) > 1e-3 * np.abs(y).max()
