"""Pins for the oracle GEMMs: exact rational products, selection matrices, symmetry.

The fp64 BLAS product is compared with an exact Fraction triple loop on tiny
non-square shapes (a transposed operand or a wrong axis changes the shape or
the values), with selection matrices whose product is known in closed form,
and with the sign / power-of-two symmetries that the quantizers preserve.
"""
import numpy as np
import pytest

from block_scaled_precision_row_amd import synthetic
from oracle import codec, dequant, gemm, quant


def bf16(v):
    return codec.f32_to_bf16(np.asarray(v, np.float64))


def _rel(a, b):
    return np.max(np.abs(np.asarray(a, float) - np.asarray(b, float))) / max(np.max(np.abs(np.asarray(b, float))), 1e-300)


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (3, 5, 32), (8, 2, 64), (2, 7, 48)])
def test_gemm_fp64_equals_exact_fraction(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    x = bf16(rng.standard_normal((M, K)))
    w = bf16(rng.standard_normal((N, K)) * 0.02)
    gw = quant.calibrate_global_scale(w)
    gx = quant.calibrate_global_scale(x)
    wq, sfw = quant.quantize_nvfp4(w, gw)
    xq, sfx = quant.quantize_nvfp4(x, gx)
    y = gemm.gemm_nvfp4(xq, sfx, gx, wq, sfw, gw)
    ex = gemm.exact_matmul(dequant.nvfp4_values(xq, sfx, gx), dequant.nvfp4_values(wq, sfw, gw))
    assert y.shape == (M, N)
    assert _rel(y, np.array([[float(v) for v in r] for r in ex])) < 1e-12
    q8x, dx = quant.quantize_fp8r(x)
    q8w, dw = quant.quantize_fp8r(w)
    y8 = gemm.gemm_fp8r(q8x, dx, q8w, dw)
    ex8 = gemm.exact_matmul(dequant.fp8r_values(q8x, dx), dequant.fp8r_values(q8w, dw))
    assert _rel(y8, np.array([[float(v) for v in r] for r in ex8])) < 1e-12


def test_tiny_workload_rows_exact():
    """Rows of the 64x256 by 128x256 weight-only workload against the exact product."""
    x = synthetic.activations(synthetic.TINY, 64, 256)
    w = synthetic.weights(synthetic.TINY, 128, 256)
    gw = quant.calibrate_global_scale(w)
    wq, sfw = quant.quantize_nvfp4(w, gw)
    y = gemm.gemm_nvfp4_weight_only(x, wq, sfw, gw)
    rows = [0, 31, 63]
    ex = gemm.exact_matmul(codec.bf16_to_f64(x[rows]), dequant.nvfp4_values(wq, sfw, gw)[:40])
    assert _rel(y[rows, :40], np.array([[float(v) for v in r] for r in ex])) < 1e-12


def test_selection_matrix_returns_weight_columns():
    """X with unit rows e_k selects columns of W^T: Y[i, n] = w_hat[n, k_i]."""
    rng = np.random.default_rng(21)
    N, K = 24, 64
    w = bf16(rng.standard_normal((N, K)) * 0.02)
    gw = quant.calibrate_global_scale(w)
    wq, sfw = quant.quantize_nvfp4(w, gw)
    ks = np.array([0, 5, 17, 63, 32])
    x = np.zeros((len(ks), K))
    x[np.arange(len(ks)), ks] = 1.0
    y = gemm.gemm_nvfp4_weight_only(bf16(x), wq, sfw, gw)
    wh = dequant.nvfp4_values(wq, sfw, gw)
    assert np.array_equal(y, wh[:, ks].T)
    q8, d8 = quant.quantize_fp8r(w)
    y8 = gemm.gemm_fp8r_weight_only(bf16(x), q8, d8)
    assert np.array_equal(y8, dequant.fp8r_values(q8, d8)[:, ks].T)


def test_symmetries_of_quantized_products():
    x = synthetic.activations(synthetic.TINY, 16, 256)
    w = synthetic.weights(synthetic.TINY, 32, 256)
    gw, gx = quant.calibrate_global_scale(w), quant.calibrate_global_scale(x)
    wq, sfw = quant.quantize_nvfp4(w, gw)
    xq, sfx = quant.quantize_nvfp4(x, gx)
    y = gemm.gemm_nvfp4(xq, sfx, gx, wq, sfw, gw)
    xn = bf16(-codec.bf16_to_f64(x))
    xqn, sfxn = quant.quantize_nvfp4(xn, gx)
    assert np.array_equal(gemm.gemm_nvfp4(xqn, sfxn, gx, wq, sfw, gw), -y)
    x2 = bf16(codec.bf16_to_f64(x) * 4)
    gx2 = quant.calibrate_global_scale(x2)
    assert gx2 == np.float32(4 * gx)
    xq2, sfx2 = quant.quantize_nvfp4(x2, gx2)
    assert np.array_equal(gemm.gemm_nvfp4(xq2, sfx2, gx2, wq, sfw, gw), 4 * y)
    q8x, dx = quant.quantize_fp8r(x)
    q8w, dw = quant.quantize_fp8r(w)
    q8n, dn = quant.quantize_fp8r(xn)
    assert np.array_equal(gemm.gemm_fp8r(q8n, dn, q8w, dw), -gemm.gemm_fp8r(q8x, dx, q8w, dw))


def test_weight_only_differs_slightly_from_fused():
    """Fallback keeps activations unquantized, so its output differs slightly from W4A4 / W8A8."""
    x = synthetic.activations(synthetic.TINY, 64, 256)
    w = synthetic.weights(synthetic.TINY, 128, 256)
    gw, gx = quant.calibrate_global_scale(w), quant.calibrate_global_scale(x)
    wq, sfw = quant.quantize_nvfp4(w, gw)
    xq, sfx = quant.quantize_nvfp4(x, gx)
    y44 = gemm.gemm_nvfp4(xq, sfx, gx, wq, sfw, gw)
    y416 = gemm.gemm_nvfp4_weight_only(x, wq, sfw, gw)
    ydense = gemm.linear_bf16(x, w)
    rel = np.linalg.norm(y44 - y416) / np.linalg.norm(y416)
    assert 0.01 < rel < 0.3
    # both quantized products stay near the unquantized bf16 product
    assert np.linalg.norm(y416 - ydense) / np.linalg.norm(ydense) < 0.2
    q8x, dx = quant.quantize_fp8r(x)
    q8w, dw = quant.quantize_fp8r(w)
    y88 = gemm.gemm_fp8r(q8x, dx, q8w, dw)
    y816 = gemm.gemm_fp8r_weight_only(x, q8w, dw)
    rel8 = np.linalg.norm(y88 - y816) / np.linalg.norm(y816)
    assert 0.001 < rel8 < 0.1
    # the materialized fallback (bf16 weights) is within bf16 rounding of weight-only
    wb = dequant.dequant_nvfp4_bf16(wq, sfw, gw)
    yfb = gemm.linear_bf16(x, wb)
    assert np.linalg.norm(yfb - y416) / np.linalg.norm(y416) < 2.0 ** -8
