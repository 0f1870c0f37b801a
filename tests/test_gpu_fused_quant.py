"""GPU parity of the W4A4 GEMM that also emits its output in nvfp4 for the next linear.

The contract is exact: the fused entry point must return the bf16 Y of
bsq_gemm_nvfp4_q bit for bit (that Y is itself held to the GEMM tolerance against
the oracle's product), and its nvfp4 encoding of Y must equal, bit for
bit, both the GPU activation quantizer and the oracle's nvfp4 quantizer ("BFL
(fp8r / nvfp4)", nvfp4 bullet) applied to that bf16 Y. Shapes cover the
256x256 and 128x128 tiled kernels, the few-token kernel and the unfused path
(K % 256 != 0 beyond the few-token range).
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
    (4096, 3072, 3072),  # 256x192 tiles
    (3100, 4000, 768),   # 256x256 tiles, ragged M and N
    (1000, 4960, 512),   # 128x128 tiles, ragged M and N
    (300, 512, 512),     # 64x64 tiles, ragged M
    (20, 1024, 512),     # few tokens
    (300, 512, 96),      # K % 256 != 0: GEMM, then the activation quantizer
    (1, 32, 32),         # smallest
]


def _bits(t):
    return host(t).view(np.uint16) if t.dtype == torch.bfloat16 else host(t)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_quantized_output_matches_gemm_then_quantizer(M, N, K):
    x = syn.normal_bf16((M, K), 54, M)
    w = syn.normal_bf16((N, K), 54, 4000 + N, sigma=0.02)
    gw = quant.calibrate_global_scale(w)
    wq, ws = quant.quantize_nvfp4(w, gw)
    gx = quant.calibrate_global_scale(x)
    xq, xs = L.bsq_quantize_act_nvfp4(dev_bf16(x), dev_scalar(gx))
    args = (xq, xs, dev_scalar(gx), dev(wq), dev(ws), dev_scalar(gw))
    y_ref = L.bsq_gemm_nvfp4_q(*args)
    torch.cuda.synchronize()
    y_host = _bits(y_ref)
    gy = quant.calibrate_global_scale(y_host)
    yq_gpu, ys_gpu = L.bsq_quantize_act_nvfp4(y_ref, dev_scalar(gy))
    yq_ora, ys_ora = quant.quantize_nvfp4(y_host, gy)

    # the bf16 Y itself against the oracle's product of the dequantized operands (X quantized by
    # the oracle; the GPU quantizer's codes equal the oracle's, checked elsewhere)
    xq_o, xs_o = quant.quantize_nvfp4(x, gx)
    assert np.array_equal(_bits(xq), xq_o) and np.array_equal(_bits(xs), xs_o)
    assert_gemm_close(y_host, gemm.gemm_nvfp4(xq_o, xs_o, gx, wq, ws, gw), "w4a4 %dx%dx%d" % (M, N, K))

    yq, ys, y = L.bsq_gemm_nvfp4_q_quantize_y(*args, dev_scalar(gy), with_y=True)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y), y_host), "bf16 output differs from bsq_gemm_nvfp4_q"
    assert np.array_equal(_bits(yq), _bits(yq_gpu)) and np.array_equal(_bits(ys), _bits(ys_gpu))
    assert np.array_equal(_bits(yq), yq_ora), "codes differ from the oracle quantizer"
    assert np.array_equal(_bits(ys), ys_ora), "block scales differ from the oracle quantizer"

    yq2, ys2, y2 = L.bsq_gemm_nvfp4_q_quantize_y(*args, dev_scalar(gy), with_y=False)
    torch.cuda.synchronize()
    assert y2 is None
    assert np.array_equal(_bits(yq2), yq_ora) and np.array_equal(_bits(ys2), ys_ora)


def test_saturating_scale():
    """A global scale far below Y's range saturates block scales at 448 and codes at +-6, as
    the quantizer does."""
    M, N, K = 64, 256, 256
    x = syn.normal_bf16((M, K), 55, M)
    w = syn.normal_bf16((N, K), 55, 5000, sigma=0.02)
    gw = quant.calibrate_global_scale(w)
    wq, ws = quant.quantize_nvfp4(w, gw)
    gx = quant.calibrate_global_scale(x)
    xq, xs = L.bsq_quantize_act_nvfp4(dev_bf16(x), dev_scalar(gx))
    args = (xq, xs, dev_scalar(gx), dev(wq), dev(ws), dev_scalar(gw))
    y_host = _bits(L.bsq_gemm_nvfp4_q(*args))
    gy = np.float32(quant.calibrate_global_scale(y_host) / 64)
    yq, ys, _ = L.bsq_gemm_nvfp4_q_quantize_y(*args, dev_scalar(gy))
    torch.cuda.synchronize()
    yq_ora, ys_ora = quant.quantize_nvfp4(y_host, gy)
    assert np.array_equal(_bits(yq), yq_ora) and np.array_equal(_bits(ys), ys_ora)
    assert (_bits(ys) == 0x7E).any()
