"""Pins for the oracle's w8a8 linear layer (per-row e4m3 quantisation and the
scaled fp8 product), against things other than the oracle itself: torch's
float8_e4m3fn rounding, exact rational arithmetic, numpy's matmul, closed
forms and the quantisation error bound against the unquantised product.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from sparse_rank_attention_amd.workloads import to_bf16_bits


def _bits(rng, shape, scale=1.0):
    return to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _rows_with_mixed_magnitudes(rng, rows, cols):
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.float32(2.0) ** rng.integers(-12, 9, size=(rows, 1)).astype(np.float32)
    x[rows // 2] = 0.0  # an all-zero row
    return to_bf16_bits(x)


def test_row_codes_are_torch_rne_of_the_scaled_row():
    rng = np.random.default_rng(1)
    xb = _rows_with_mixed_magnitudes(rng, 37, 200)
    codes, scale, deq = oracle.quant_rows_e4m3(xb)
    x = oracle.widen_bf16(xb).astype(np.float32)
    for m in range(x.shape[0]):
        amax = np.float32(np.abs(x[m]).max())
        if amax == 0:
            assert scale[m] == 1.0 and not codes[m].any() and not deq[m].any()
            continue
        y = torch.from_numpy(x[m] * (np.float32(448.0) / amax))  # fp32 product
        ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(codes[m], ref)
        assert scale[m] == np.float32(amax / np.float32(448.0))
        # the largest element lands on the top code
        assert (codes[m] & 0x7F).max() == 0x7E
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(deq, vals * scale[:, None].astype(np.float64))


def test_row_scale_is_per_row_and_power_of_two_equivariant():
    """Scaling one row by 2^e (exact in bf16) leaves every code unchanged and
    multiplies only that row's scale by 2^e."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((8, 96)).astype(np.float32)
    c0, s0, _ = oracle.quant_rows_e4m3(to_bf16_bits(x))
    x2 = x.copy()
    x2[3] *= np.float32(2.0 ** -7)
    x2[5] *= np.float32(2.0 ** 6)
    c1, s1, _ = oracle.quant_rows_e4m3(to_bf16_bits(x2))
    np.testing.assert_array_equal(c0, c1)
    expect = s0.copy()
    expect[3] *= np.float32(2.0 ** -7)
    expect[5] *= np.float32(2.0 ** 6)
    np.testing.assert_array_equal(s1, expect)


def test_row_round_trip_within_half_an_e4m3_step():
    rng = np.random.default_rng(3)
    xb = _rows_with_mixed_magnitudes(rng, 64, 300)
    _, scale, deq = oracle.quant_rows_e4m3(xb)
    x = oracle.widen_bf16(xb)
    sc = scale[:, None].astype(np.float64)
    # normals: 3 mantissa bits (half step 2^-4 relative); subnormals: spacing 2^-9
    bound = 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * sc + 1e-6 * np.abs(x)
    assert np.all(np.abs(deq - x) <= bound)


def test_gemm_dot_is_exact_rational():
    rng = np.random.default_rng(4)
    M, N, K = 3, 5, 64
    a = rng.integers(0, 256, (M, K), dtype=np.uint8)
    w = rng.integers(0, 256, (N, K), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0  # no NaN codes
    w[(w & 0x7F) == 0x7F] = 0
    val = lambda c: Fraction(float(torch.tensor([int(c)], dtype=torch.uint8).view(torch.float8_e4m3fn)
                                   .to(torch.float64)))
    y = oracle.gemm_w8a8(a, np.ones(M), w, np.ones(N))
    for m in range(M):
        for n in range(N):
            exact = sum(val(a[m, k]) * val(w[n, k]) for k in range(K))
            assert Fraction(y[m, n]) == exact


def test_gemm_matches_numpy_on_dequantised_operands():
    """Non-square, ragged sizes with distinct per-row and per-column scales and
    a bias: y = (deq a) (deq w)^T + bias."""
    rng = np.random.default_rng(5)
    M, N, K = 45, 29, 192
    ca, sa, da = oracle.quant_rows_e4m3(_rows_with_mixed_magnitudes(rng, M, K))
    cw, sw, dw = oracle.quant_rows_e4m3(_bits(rng, (N, K), 0.05))
    bias = rng.standard_normal(N).astype(np.float32)
    y, yabs = oracle.gemm_w8a8(ca, sa, cw, sw, bias, with_abs=True)
    ref = da @ dw.T + bias.astype(np.float64)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    ref_abs = np.abs(da) @ np.abs(dw).T + np.abs(bias).astype(np.float64)
    np.testing.assert_allclose(yabs, ref_abs, rtol=1e-12)
    assert np.all(yabs >= np.abs(y) * (1 - 1e-12))
    # without a bias
    np.testing.assert_allclose(oracle.gemm_w8a8(ca, sa, cw, sw), da @ dw.T, rtol=1e-12,
                               atol=1e-12 * np.abs(ref).max())


def test_gemm_with_unit_weights_returns_the_dequantised_activations():
    rng = np.random.default_rng(6)
    M, K = 20, 128
    ca, sa, da = oracle.quant_rows_e4m3(_bits(rng, (M, K)))
    w = np.zeros((K, K), dtype=np.uint8)
    np.fill_diagonal(w, 0x38)  # e4m3 1.0
    y = oracle.gemm_w8a8(ca, sa, w, np.ones(K, dtype=np.float32))
    np.testing.assert_array_equal(y, da)


@pytest.mark.parametrize("K", [64, 512])
def test_linear_within_quantisation_bound_of_unquantised_product(K):
    rng = np.random.default_rng(7 + K)
    M, N = 33, 40
    xb = _bits(rng, (M, K))
    wb = _bits(rng, (N, K), 1 / np.sqrt(K))
    bias = rng.standard_normal(N).astype(np.float32)
    y = oracle.linear_w8a8(xb, wb, bias)
    x, w = oracle.widen_bf16(xb), oracle.widen_bf16(wb)
    exact = x @ w.T + bias.astype(np.float64)
    _, sx, _ = oracle.quant_rows_e4m3(xb)
    _, swt, _ = oracle.quant_rows_e4m3(wb)
    ex = 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * sx[:, None] + 1e-6 * np.abs(x)
    ew = 2.0 ** -4 * np.abs(w) + 2.0 ** -10 * swt[:, None] + 1e-6 * np.abs(w)
    bound = np.abs(x) @ ew.T + ex @ np.abs(w).T + ex @ ew.T
    err = np.abs(y - exact)
    assert np.all(err <= bound)
    # and the error is real quantisation error, not zero
    assert err.max() > 0
