"""GPU parity of the linears that hand their output to the next quantized linear already
encoded, in either format ("BFL (fp8r / nvfp4)": every quantized linear quantizes its input
at run time -- fp8r per row to E4M3, nvfp4 per 16-block with its input_scale).

The contract is exact: the bf16 Y must equal, bit for bit, the plain GEMM entry point's
(and stay within the GEMM tolerance of the oracle's product), and the encoding must equal,
bit for bit, the oracle's quantizer (and the GPU activation quantizer) applied to that bf16
Y. Shapes take every route: the tiled kernels' tile shapes with ragged edges and a partial
last 64-column segment (N % 64 == 32), the few-token kernels, the W4A4 decode kernel
(K % 256 != 0) and rows longer than the encode pass's one-workgroup limit.
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_row_amd import synthetic as syn
from oracle import gemm, quant
from tests.gpu_util import assert_gemm_close, dev, dev_bf16, dev_scalar, host

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from block_scaled_precision_row_amd import _lib as L

SHAPES = [
    (4096, 3072, 3072),  # 256 x 192 tiles
    (3100, 4000, 768),   # 256 x 256 tiles, ragged M, N % 64 == 32
    (1000, 4960, 512),   # 128 x 128 tiles, ragged M and N
    (300, 512, 512),     # 64 x 64 tiles, ragged M
    (2048, 3040, 512),   # fp8r: 128 x 128 tiles two to a compute unit, N % 64 == 32
    (20, 1024, 512),     # few tokens
    (64, 16416, 256),    # rows longer than 16384 values (the encode pass reads Y for the maximum)
    (1, 32, 32),         # smallest
]


def _bits(t):
    return host(t).view(np.uint16) if t.dtype == torch.bfloat16 else host(t)


def _check_encoding(yq, ys, y_host, fmt, gy=None):
    if fmt == "fp8r":
        q_ref, d_ref = quant.quantize_fp8r(y_host)
        assert np.array_equal(_bits(yq), q_ref), "fp8r codes differ from the oracle quantizer"
        assert np.array_equal(_bits(ys).view(np.uint32), d_ref.view(np.uint32)), "fp8r row scales differ"
        q_gpu, d_gpu = L.bsq_quantize_act_fp8r(dev_bf16(y_host))
        assert np.array_equal(_bits(yq), _bits(q_gpu)) and np.array_equal(_bits(ys), _bits(d_gpu))
    else:
        q_ref, s_ref = quant.quantize_nvfp4(y_host, gy)
        assert np.array_equal(_bits(yq), q_ref), "nvfp4 codes differ from the oracle quantizer"
        assert np.array_equal(_bits(ys), s_ref), "nvfp4 block scales differ"


@pytest.mark.parametrize("fmt", ["fp8r", "nvfp4"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_fp8r_linear_with_quantized_output(M, N, K, fmt):
    print("fp8r producer -> %s M=%d N=%d K=%d" % (fmt, M, N, K), flush=True)
    x = syn.normal_bf16((M, K), 56, M, outlier_frac=0.01)
    w = syn.normal_bf16((N, K), 56, 4000 + N, sigma=0.02)
    wq, sw = quant.quantize_fp8r(w)
    xq, sx = L.bsq_quantize_act_fp8r(dev_bf16(x))
    args = (xq, sx, dev(wq), dev(sw))
    y_plain = _bits(L.bsq_gemm_fp8r_q(*args))
    torch.cuda.synchronize()
    rows = np.arange(M) if M <= 1024 else np.arange(0, M, 8)
    xq_o, sx_o = quant.quantize_fp8r(x[rows])
    assert_gemm_close(y_plain[rows], gemm.gemm_fp8r(xq_o, sx_o, wq, sw), "fp8r %dx%dx%d" % (M, N, K))
    out = L.BSQ_FMT_FP8R if fmt == "fp8r" else L.BSQ_FMT_NVFP4
    gy = None if fmt == "fp8r" else quant.calibrate_global_scale(y_plain)
    gyd = None if gy is None else dev_scalar(gy)
    for with_y in (True, False):
        yq, ys, y = L.bsq_gemm_fp8r_q_quantize_y(*args, out, gyd, with_y=with_y)
        torch.cuda.synchronize()
        if with_y:
            assert np.array_equal(_bits(y), y_plain), "bf16 output differs from bsq_gemm_fp8r_q"
        else:
            assert y is None
        _check_encoding(yq, ys, y_plain, fmt, gy)


@pytest.mark.parametrize("M,N,K", SHAPES + [(300, 512, 96), (2048, 3072, 1056)])
def test_w4a4_linear_with_fp8r_output(M, N, K):
    print("W4A4 producer -> fp8r M=%d N=%d K=%d" % (M, N, K), flush=True)
    x = syn.normal_bf16((M, K), 57, M)
    w = syn.normal_bf16((N, K), 57, 4000 + N, sigma=0.02)
    gw = quant.calibrate_global_scale(w)
    wq, ws = quant.quantize_nvfp4(w, gw)
    gx = quant.calibrate_global_scale(x)
    xq, xs = L.bsq_quantize_act_nvfp4(dev_bf16(x), dev_scalar(gx))
    args = (xq, xs, dev_scalar(gx), dev(wq), dev(ws), dev_scalar(gw))
    y_plain = _bits(L.bsq_gemm_nvfp4_q(*args))
    torch.cuda.synchronize()
    for with_y in (True, False):
        yq, yd, y = L.bsq_gemm_nvfp4_q_quantize_y_fp8r(*args, with_y=with_y)
        torch.cuda.synchronize()
        if with_y:
            assert np.array_equal(_bits(y), y_plain), "bf16 output differs from bsq_gemm_nvfp4_q"
        _check_encoding(yq, yd, y_plain, "fp8r")


def test_fp8r_output_of_rows_with_zeros_and_one_large_value():
    """Rows that are all zero (scale 0, signed-zero codes) and rows whose maximum sits in one
    segment far from the others: the row scale must come from the whole row."""
    M, N, K = 256, 3072, 256
    x = syn.normal_bf16((M, K), 58, M)
    xv = (x.astype(np.uint32) << 16).view(np.float32)
    xv[::7] = 0.0                       # zero rows of X give zero rows of Y
    x = (xv.view(np.uint32) >> 16).astype(np.uint16)
    w = syn.normal_bf16((N, K), 58, 4000 + N, sigma=0.02)
    wv = (w.astype(np.uint32) << 16).view(np.float32)
    wv[2900] *= 64.0                    # one output column far larger than the rest
    w = (wv.view(np.uint32) >> 16).astype(np.uint16)
    wq, sw = quant.quantize_fp8r(w)
    xq, sx = L.bsq_quantize_act_fp8r(dev_bf16(x))
    args = (xq, sx, dev(wq), dev(sw))
    y_plain = _bits(L.bsq_gemm_fp8r_q(*args))
    yq, yd, _ = L.bsq_gemm_fp8r_q_quantize_y(*args, L.BSQ_FMT_FP8R, None)
    torch.cuda.synchronize()
    _check_encoding(yq, yd, y_plain, "fp8r")
    assert np.all(_bits(yd)[::7] == 0)


# Weight-only producers (bf16 activations): the tiled weight-only kernels (256 x 192 and 128 x 128
# nvfp4 tiles, 128 x 256 E4M3 tiles at these sizes), the few-token kernels, and for nvfp4 weights
# with K % 64 != 0 the decode GEMM (the last three run the GEMM, then the quantizer).
WO_SHAPES = [(4096, 3072, 3072), (1000, 4960, 512), (300, 544, 512), (20, 1024, 512), (300, 512, 96), (1, 32, 32)]


@pytest.mark.parametrize("fmt", ["fp8r", "nvfp4"])
@pytest.mark.parametrize("wfmt", ["fp8r", "nvfp4"])
@pytest.mark.parametrize("M,N,K", WO_SHAPES)
def test_weight_only_linear_with_quantized_output(M, N, K, wfmt, fmt):
    print("weight-only %s producer -> %s M=%d N=%d K=%d" % (wfmt, fmt, M, N, K), flush=True)
    x = syn.normal_bf16((M, K), 59, M, outlier_frac=0.01)
    w = syn.normal_bf16((N, K), 59, 4000 + N, sigma=0.02)
    dx = dev_bf16(x)
    rows = np.arange(M) if M <= 1024 else np.arange(0, M, 8)
    if wfmt == "fp8r":
        wq, sw = quant.quantize_fp8r(w)
        wargs = (L.BSQ_FMT_FP8R, dx, dev(wq), dev(sw), None)
        y_plain = _bits(L.bsq_gemm_fp8r(dx, dev(wq), dev(sw), flags=L.BSQ_WEIGHT_ONLY))
        ref = gemm.gemm_fp8r_weight_only(x[rows], wq, sw)
    else:
        gw = quant.calibrate_global_scale(w)
        wq, ws = quant.quantize_nvfp4(w, gw)
        wargs = (L.BSQ_FMT_NVFP4, dx, dev(wq), dev(ws), dev_scalar(gw))
        y_plain = _bits(L.bsq_gemm_nvfp4(dx, dev(wq), dev(ws), dev_scalar(gw), None, flags=L.BSQ_WEIGHT_ONLY))
        ref = gemm.gemm_nvfp4_weight_only(x[rows], wq, ws, gw)
    torch.cuda.synchronize()
    assert_gemm_close(y_plain[rows], ref, "weight-only %s %dx%dx%d" % (wfmt, M, N, K))
    out = L.BSQ_FMT_FP8R if fmt == "fp8r" else L.BSQ_FMT_NVFP4
    gy = None if fmt == "fp8r" else quant.calibrate_global_scale(y_plain)
    gyd = None if gy is None else dev_scalar(gy)
    for with_y in (True, False):
        yq, ys, y = L.bsq_gemm_weight_only_quantize_y(*wargs, out, gyd, with_y=with_y)
        torch.cuda.synchronize()
        if with_y:
            assert np.array_equal(_bits(y), y_plain), "bf16 output differs from the weight-only linear"
        else:
            assert y is None
        _check_encoding(yq, ys, y_plain, fmt, gy)


def test_weight_only_quantized_output_strided_input():
    """x with a row pitch wider than K (a view of a wider matrix), on the tiled route."""
    M, N, K = 1024, 3072, 512
    full = syn.normal_bf16((M, K + 64), 60, M)
    w = syn.normal_bf16((N, K), 60, 4000 + N, sigma=0.02)
    wq, sw = quant.quantize_fp8r(w)
    dx = dev_bf16(full)[:, :K]
    y_plain = _bits(L.bsq_gemm_fp8r(dx, dev(wq), dev(sw), flags=L.BSQ_WEIGHT_ONLY))
    yq, yd, y = L.bsq_gemm_weight_only_quantize_y(L.BSQ_FMT_FP8R, dx, dev(wq), dev(sw), None, L.BSQ_FMT_FP8R, None,
                                                  with_y=True)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y), y_plain)
    _check_encoding(yq, yd, y_plain, "fp8r")
