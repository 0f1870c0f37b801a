"""GPU parity over a seeded sweep of ragged shapes, all four schemes of the linear.

The GEMM entry points pick their kernel from the shape (few-token kernels, the
64 x 64 / 64 x 128 / 128 x 128 small-grid tiles, the large tiles, the
weight-only tiled kernel, the decode-GEMM fallback for K % 256 != 0 or
K % 64 != 0), so a sweep over M, N and K that crosses those boundaries checks
every route against the oracle with the same tolerance as test_gpu_gemm.py.
Shapes stay small enough that the oracle's fp64 products take seconds. A second
sweep attaches a LoRA adapter of random rank to every scheme; a third runs grids of
several rounds of large tiles (up to about 6000 x 7000), compared on sampled rows.
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_row_amd import synthetic as syn
from oracle import gemm, lora, quant
from tests.gpu_util import assert_gemm_close, dev, dev_bf16, dev_scalar, host

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from block_scaled_precision_row_amd import _lib as L

K_CHOICES = [32, 64, 96, 128, 160, 256, 288, 512, 544, 1024, 1056]


def _shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.choice([int(rng.integers(1, 33)), int(rng.integers(33, 300)), int(rng.integers(300, 700))]))
        N = int(rng.integers(1, 900))
        K = int(rng.choice(K_CHOICES))
        out.append((M, N, K))
    return out


SHAPES = _shapes(48, 20260101)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_every_scheme_on_a_ragged_shape(M, N, K):
    x = syn.normal_bf16((M, K), 63, M * 1009 + N * 7 + K, outlier_frac=0.01)
    w = syn.normal_bf16((N, K), 63, 9100 + N * 13 + K, sigma=0.02)
    dx = dev_bf16(x)
    tag = "%dx%dx%d" % (M, N, K)

    wq, sw = quant.quantize_fp8r(w)
    y8 = host(L.bsq_gemm_fp8r(dx, dev(wq), dev(sw)))
    y8w = host(L.bsq_gemm_fp8r(dx, dev(wq), dev(sw), flags=L.BSQ_WEIGHT_ONLY))
    gw = quant.calibrate_global_scale(w)
    wp, sfw = quant.quantize_nvfp4(w, gw)
    gx = quant.calibrate_global_scale(x)
    y4 = host(L.bsq_gemm_nvfp4(dx, dev(wp), dev(sfw), dev_scalar(gw), dev_scalar(gx)))
    y4w = host(L.bsq_gemm_nvfp4(dx, dev(wp), dev(sfw), dev_scalar(gw), None, flags=L.BSQ_WEIGHT_ONLY))
    torch.cuda.synchronize()

    xq, sx = quant.quantize_fp8r(x)
    assert_gemm_close(y8, gemm.gemm_fp8r(xq, sx, wq, sw), "w8a8 " + tag)
    assert_gemm_close(y8w, gemm.gemm_fp8r_weight_only(x, wq, sw), "w8a16 " + tag)
    xp, sfx = quant.quantize_nvfp4(x, gx)
    assert_gemm_close(y4, gemm.gemm_nvfp4(xp, sfx, gx, wp, sfw, gw), "w4a4 " + tag)
    assert_gemm_close(y4w, gemm.gemm_nvfp4_weight_only(x, wp, sfw, gw), "w4a16 " + tag)


LORA_SHAPES = [(M, N, K, int(r)) for (M, N, K), r in
               zip(_shapes(12, 20260202), np.random.default_rng(20260203).integers(1, 129, 12))]


@pytest.mark.parametrize("M,N,K,rank", LORA_SHAPES)
def test_every_scheme_with_an_adapter_on_a_ragged_shape(M, N, K, rank):
    from tests.test_gpu_lora import t_rounding_bound

    x = syn.normal_bf16((M, K), 64, M * 1013 + N * 5 + K)
    w = syn.normal_bf16((N, K), 64, 9200 + N * 11 + K, sigma=0.02)
    a, b = syn.lora_adapter(64, rank, N, K, block=M % 7)
    scale = 0.75
    dx, da, db = dev_bf16(x), dev_bf16(a), dev_bf16(b)
    extra = t_rounding_bound(x, a, b, scale)
    tag = "%dx%dx%d r%d" % (M, N, K, rank)
    wq, sw = quant.quantize_fp8r(w)
    gw = quant.calibrate_global_scale(w)
    wp, sfw = quant.quantize_nvfp4(w, gw)
    gx = quant.calibrate_global_scale(x)
    xq, sx = quant.quantize_fp8r(x)
    xp, sfx = quant.quantize_nvfp4(x, gx)
    runs = [
        ("w8a8", L.bsq_gemm_fp8r_lora(dx, dev(wq), dev(sw), da, db, scale), gemm.gemm_fp8r(xq, sx, wq, sw)),
        ("w8a16", L.bsq_gemm_fp8r_lora(dx, dev(wq), dev(sw), da, db, scale, flags=L.BSQ_WEIGHT_ONLY),
         gemm.gemm_fp8r_weight_only(x, wq, sw)),
        ("w4a4", L.bsq_gemm_nvfp4_lora(dx, dev(wp), dev(sfw), dev_scalar(gw), dev_scalar(gx), da, db, scale),
         gemm.gemm_nvfp4(xp, sfx, gx, wp, sfw, gw)),
        ("w4a16", L.bsq_gemm_nvfp4_lora(dx, dev(wp), dev(sfw), dev_scalar(gw), None, da, db, scale,
                                        flags=L.BSQ_WEIGHT_ONLY),
         gemm.gemm_nvfp4_weight_only(x, wp, sfw, gw)),
    ]
    torch.cuda.synchronize()
    for name, y, base in runs:
        assert_gemm_close(host(y), lora.lora_linear(base, x, a, b, scale), name + " " + tag, extra=extra)


def _large_shapes(n, seed):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(700, 6000)), int(rng.integers(900, 7000)), int(rng.choice([256, 512, 768, 1024, 1088, 1536])))
            for _ in range(n)]


LARGE_SHAPES = _large_shapes(8, 20260303)


@pytest.mark.parametrize("M,N,K", LARGE_SHAPES)
def test_every_scheme_on_a_large_ragged_grid(M, N, K):
    """Grids of several rounds of large tiles, where the launchers choose among 256 x 256, 256 x 192,
    128 x 128 (fp8r, W4A4) and the weight-only tiles by whole rounds: every scheme against the
    oracle on sampled rows (the first and last row always among them)."""
    from tests.test_gpu_gemm import run_fp8r, run_nvfp4

    x = syn.normal_bf16((M, K), 65, M * 7 + N + K, outlier_frac=0.01)
    w = syn.normal_bf16((N, K), 65, 9300 + N * 3 + K, sigma=0.02)
    tag = "%dx%dx%d" % (M, N, K)
    run_fp8r(x, w, sample=48, what="w8a8 " + tag)
    run_fp8r(x, w, weight_only=True, sample=48, what="w8a16 " + tag)
    run_nvfp4(x, w, sample=48, what="w4a4 " + tag)
    run_nvfp4(x, w, weight_only=True, sample=48, what="w4a16 " + tag)
