"""GPU test of bsq_gemm_fp8r_noalloc: the fp8r linear on the library's own device scratch.

Called through the C ABI (ctypes). Its output must equal bsq_gemm_fp8r's bit for bit (the
same kernels on the same inputs; that entry point is itself held to the oracle elsewhere, and
the first case here is also checked against the oracle's product), on two calls in a row where
the second is smaller than the first, so that nothing of the first call's scratch contents
leaks into the second. A shape beyond the scratch is refused before anything is enqueued.
"""
import ctypes

import numpy as np
import pytest
import torch

from block_scaled_precision_row_amd import synthetic as syn
from oracle import gemm, quant
from tests.gpu_util import assert_gemm_close, dev, dev_bf16, host

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from block_scaled_precision_row_amd import _lib as L


def _linear(M, N, K, seed):
    x = syn.normal_bf16((M, K), seed, M, outlier_frac=0.01)
    w = syn.normal_bf16((N, K), seed, 1000 + N, sigma=0.02)
    wq, sw = quant.quantize_fp8r(w)
    return x, wq, sw


def _noalloc(xd, wd, swd, M, N, K, flags=0):
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = L.lib.bsq_gemm_fp8r_noalloc(P(xd), K, P(wd), P(swd), P(y), N, M, N, K, flags,
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, L.STATUS.get(st, st)
    return y


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    cases = [(2048, 3072, 3072, 90), (300, 1000, 512, 91)]   # the second call is smaller
    outs = []
    for M, N, K, seed in cases:
        print("noalloc case M=%d N=%d K=%d" % (M, N, K), flush=True)
        x, wq, sw = _linear(M, N, K, seed)
        xd, wd, swd = dev_bf16(x), dev(wq), dev(sw)
        y0 = _noalloc(xd, wd, swd, M, N, K)
        y1 = L.bsq_gemm_fp8r(xd, wd, swd)
        torch.cuda.synchronize()
        assert np.array_equal(host(y0), host(y1)), (M, N, K)
        outs.append((M, N, K, x, wq, sw, host(y0)))
    M, N, K, x, wq, sw, y = outs[0]
    rows = np.arange(0, M, 16)
    xq, sx = quant.quantize_fp8r(x[rows])
    assert_gemm_close(y[rows], gemm.gemm_fp8r(xq, sx, wq, sw), "noalloc fp8r %dx%dx%d" % (M, N, K))


def test_noalloc_weight_only_and_refusals():
    M, N, K = 64, 256, 512
    x, wq, sw = _linear(M, N, K, 92)
    xd, wd, swd = dev_bf16(x), dev(wq), dev(sw)
    y0 = _noalloc(xd, wd, swd, M, N, K, flags=L.BSQ_WEIGHT_ONLY)
    y1 = L.bsq_gemm_fp8r(xd, wd, swd, flags=L.BSQ_WEIGHT_ONLY)
    torch.cuda.synchronize()
    assert np.array_equal(host(y0), host(y1))
    # beyond the scratch: refused on the host (pointers are never touched)
    big_m = L.BSQ_NOALLOC_MAX_BYTES // 4096 + 1
    P = ctypes.c_void_p
    st = L.lib.bsq_gemm_fp8r_noalloc(P(1 << 20), 4096, P(1 << 21), P(1 << 22), P(1 << 23), 64, big_m, 64, 4096, 0,
                                     None)
    assert st == 4   # BSQ_ERR_WORKSPACE
