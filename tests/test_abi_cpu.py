"""CPU checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments on the host before any HIP call.

Pointers passed here are fake (never dereferenced): every call below fails
validation before touching the device. The one call with valid arguments is
only made when no GPU is present, where it must report BSQ_ERR_DEVICE.
"""
import ctypes
import os
import re

import pytest
import torch

from block_scaled_precision_row_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
L = _lib.lib
P = ctypes.c_void_p
A = P(1 << 20)       # fake, 16-byte aligned
B = P((1 << 20) + 4096)
C = P((1 << 20) + 8192)
D = P((1 << 20) + 12288)
ODD = P((1 << 20) + 2)
OK, NULL, SHAPE, ALIGN, WS, DEV, HIP, ARG = range(8)


def declared_symbols():
    with open(os.path.join(ROOT, "include", "bsq.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(bsq_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound():
    syms = declared_symbols()
    assert len(syms) == 27
    so = ctypes.CDLL(_lib.LIB_PATH)
    for s in syms:
        assert hasattr(so, s), s
        assert s in _lib.SIGNATURES, s
    assert L.bsq_abi_version() == 3
    assert L.bsq_status_string(SHAPE).decode().startswith("invalid shape")


def test_weight_only_quantized_output_validation():
    fp8, nv = _lib.BSQ_FMT_FP8R, _lib.BSQ_FMT_NVFP4
    g = L.bsq_gemm_weight_only_quantize_y
    ws = L.bsq_gemm_quantize_y_workspace_bytes(fp8, 64, 64, 0)
    # w_fmt, x, ldx, w, w_scale, w_scale2, out_fmt, y_global, yq, yq_scale, y, ldy, M, N, K, ws, ws_bytes, stream
    assert g(3, A, 64, B, C, None, fp8, None, A, B, None, 0, 64, 64, 64, A, ws, None) == ARG     # weight format
    assert g(fp8, A, 64, B, C, D, fp8, None, A, B, None, 0, 64, 64, 64, A, ws, None) == ARG      # fp8r: no scale2
    assert g(nv, A, 64, B, C, None, fp8, None, A, B, None, 0, 64, 64, 64, A, ws, None) == NULL   # nvfp4: scale2
    assert g(fp8, A, 64, B, None, None, fp8, None, A, B, None, 0, 64, 64, 64, A, ws, None) == NULL  # w_scale
    assert g(fp8, A, 64, B, C, None, 3, None, A, B, None, 0, 64, 64, 64, A, ws, None) == ARG     # output format
    assert g(fp8, A, 64, B, C, None, nv, None, A, B, None, 0, 64, 64, 64, A, ws, None) == NULL   # nvfp4 out: global
    assert g(fp8, A, 64, B, C, None, fp8, None, A, B, None, 0, 64, 48, 64, A, ws, None) == SHAPE  # N % 32
    assert g(fp8, A, 60, B, C, None, fp8, None, A, B, None, 0, 64, 64, 64, A, ws, None) == SHAPE  # ldx < K
    assert g(fp8, A, 64, B, C, None, fp8, None, ODD, B, None, 0, 64, 64, 64, A, ws, None) == ALIGN  # yq
    assert g(fp8, A, 64, B, C, None, fp8, None, A, B, None, 0, 64, 64, 64, A, ws - 1, None) == WS
    assert g(fp8, None, 64, None, None, None, fp8, None, None, None, None, 0, 0, 64, 64, None, 0, None) == OK  # empty


def test_grouped_validation():
    fp8, nv = _lib.BSQ_FMT_FP8R, _lib.BSQ_FMT_NVFP4
    g = L.bsq_gemm_grouped_q
    GP = _lib.GemmProblem

    def probs(*ps):
        arr = (GP * len(ps))()
        for i, p in enumerate(ps):
            arr[i] = p
        return arr

    f8 = GP(A.value, B.value, None, C.value, D.value, None, A.value, 64, 64, 64, 128)  # xq, sx, w, sw, y
    n4 = GP(A.value, B.value, C.value, C.value, D.value, D.value, A.value, 64, 64, 64, 256)
    assert g(3, probs(f8), 1, None) == ARG                       # format
    assert g(fp8, probs(f8), -1, None) == ARG                    # count
    assert g(fp8, probs(*[f8] * 9), 9, None) == ARG              # more than BSQ_MAX_GROUP
    assert g(fp8, None, 0, None) == OK                           # nothing to do
    assert g(fp8, None, 2, None) == NULL                         # no descriptors
    bad = GP(A.value, B.value, C.value, C.value, D.value, None, A.value, 64, 64, 64, 128)
    assert g(fp8, probs(f8, bad), 2, None) == ARG                # fp8r takes no input_scale
    assert g(nv, probs(n4, GP(A.value, B.value, None, C.value, D.value, D.value, A.value, 64, 64, 64, 256)),
             2, None) == NULL                                    # nvfp4 needs input_scale
    assert g(fp8, probs(f8, GP(A.value, B.value, None, C.value, D.value, None, A.value, 64, 64, 64, 100)),
             2, None) == SHAPE                                   # K % 32
    assert g(fp8, probs(f8, GP(A.value, None, None, C.value, D.value, None, A.value, 64, 64, 64, 128)),
             2, None) == NULL                                    # x_scale
    assert g(nv, probs(n4, GP(ODD.value, B.value, C.value, C.value, D.value, D.value, A.value, 64, 64, 64, 256)),
             2, None) == ALIGN                                   # xq
    assert g(fp8, probs(f8, GP(A.value, B.value, None, C.value, D.value, None, A.value, 32, 64, 64, 128)),
             2, None) == SHAPE                                   # ldy < N
    # empty problems are skipped without looking at their pointers; all empty is a no-op
    empty = GP(None, None, None, None, None, None, None, 64, 0, 64, 128)  # M = 0
    assert g(fp8, probs(empty, empty), 2, None) == OK
    # a bad problem after a valid one still fails before anything is enqueued (no device here)
    assert g(fp8, probs(f8, GP(A.value, B.value, None, C.value, D.value, None, A.value, 64, 64, 64, 0)),
             2, None) == SHAPE
    if not torch.cuda.is_available():
        assert g(fp8, probs(f8, f8), 2, None) == DEV
    with pytest.raises(ValueError):
        _lib.bsq_gemm_grouped_q(fp8, [None] * 9)


def test_grouped_weight_only_validation():
    fp8, nv = _lib.BSQ_FMT_FP8R, _lib.BSQ_FMT_NVFP4
    g = L.bsq_gemm_grouped_weight_only
    WP = _lib.WeightOnlyProblem

    def probs(*ps):
        arr = (WP * len(ps))()
        for i, p in enumerate(ps):
            arr[i] = p
        return arr

    # x, ldx, w, w_scale, w_scale2, y, ldy, M, N, K
    f8 = WP(A.value, 128, B.value, C.value, None, D.value, 64, 16, 64, 128)
    n4 = WP(A.value, 256, B.value, C.value, D.value, A.value, 64, 16, 64, 256)
    assert g(3, probs(f8), 1, None) == ARG                                   # format
    assert g(fp8, probs(f8), 9, None) == ARG                                 # more than BSQ_MAX_GROUP
    assert g(fp8, probs(f8), -1, None) == ARG
    assert g(fp8, None, 0, None) == OK and g(fp8, None, 1, None) == NULL
    assert g(fp8, probs(f8, WP(A.value, 128, B.value, C.value, D.value, D.value, 64, 16, 64, 128)), 2, None) == ARG
    assert g(nv, probs(n4, WP(A.value, 256, B.value, C.value, None, A.value, 64, 16, 64, 256)), 2, None) == NULL
    assert g(fp8, probs(f8, WP(A.value, 120, B.value, C.value, None, D.value, 64, 16, 64, 128)), 2, None) == SHAPE
    assert g(fp8, probs(f8, WP(ODD.value, 128, B.value, C.value, None, D.value, 64, 16, 64, 128)), 2, None) == ALIGN
    assert g(nv, probs(n4, WP(A.value, 256, B.value, ODD.value, D.value, A.value, 64, 16, 64, 256)), 2, None) == ALIGN
    empty = WP(None, 128, None, None, None, None, 64, 0, 64, 128)  # M = 0: skipped unread
    assert g(fp8, probs(empty, empty), 2, None) == OK
    if not torch.cuda.is_available():
        assert g(fp8, probs(f8, f8), 2, None) == DEV
    with pytest.raises(ValueError):
        _lib.bsq_gemm_grouped_weight_only(fp8, [None] * 9)


def test_workspace_sizes():
    pad = lambda n: (n + 255) // 256 * 256
    assert L.bsq_gemm_workspace_bytes(_lib.BSQ_FMT_FP8R, 4096, 3072, 3072, 0) == pad(4096 * 3072) + pad(4 * 4096)
    assert L.bsq_gemm_workspace_bytes(_lib.BSQ_FMT_NVFP4, 4096, 12288, 3072, 0) == pad(4096 * 1536) + pad(4096 * 192)
    assert L.bsq_gemm_workspace_bytes(_lib.BSQ_FMT_NVFP4, 4096, 12288, 3072, _lib.BSQ_WEIGHT_ONLY) == 0
    assert L.bsq_gemm_workspace_bytes(_lib.BSQ_FMT_FP8R, 0, 1, 32, 0) == 0
    assert L.bsq_calibrate_workspace_bytes(4096, 3072) == 4096


def test_quantizer_validation():
    q = L.bsq_quantize_act_fp8r
    assert q(A, 4, 48, 48, B, C, None) == SHAPE          # K % 32
    assert q(A, 4, 64, 32, B, C, None) == SHAPE          # ldx < K
    assert q(A, 4, 64, 68, B, C, None) == SHAPE          # ldx % 8
    assert q(A, -1, 64, 64, B, C, None) == SHAPE
    assert q(A, 4, 0, 64, B, C, None) == SHAPE
    assert q(None, 4, 64, 64, B, C, None) == NULL
    assert q(ODD, 4, 64, 64, B, C, None) == ALIGN
    assert q(None, 0, 64, 64, None, None, None) == OK    # empty: nothing to do
    n = L.bsq_quantize_act_nvfp4
    assert n(A, 4, 64, 64, None, B, C, None) == NULL
    assert n(A, 4, 64, 64, D, ODD, C, None) == ALIGN
    assert n(A, 4, 40, 64, D, B, C, None) == SHAPE
    assert n(None, 0, 64, 64, None, None, None, None) == OK
    c = L.bsq_calibrate_global_scale
    assert c(A, 0, 64, 64, B, C, 4096, None) == SHAPE
    assert c(A, 4, 64, 64, B, None, 4096, None) == WS
    assert c(A, 4, 64, 64, B, C, 0, None) == WS


def test_gemm_validation():
    g = L.bsq_gemm_fp8r
    ws = L.bsq_gemm_workspace_bytes(_lib.BSQ_FMT_FP8R, 64, 64, 64, 0)
    assert g(A, 64, B, C, D, 64, 64, 64, 64, 0, None, 0, None) == WS
    assert g(A, 64, B, C, D, 64, 64, 64, 64, 0, A, ws - 1, None) == WS
    assert g(A, 64, B, C, D, 64, 64, 64, 64, 2, A, ws, None) == ARG
    assert g(A, 64, B, None, D, 64, 64, 64, 64, 0, A, ws, None) == NULL
    assert g(A, 64, B, C, D, 63, 64, 64, 64, 0, A, ws, None) == SHAPE   # ldy < N
    assert g(A, 64, B, C, D, 64, 64, 64, 48, 0, A, ws, None) == SHAPE   # K % 32
    assert g(A, 64, ODD, C, D, 64, 64, 64, 64, 0, A, ws, None) == ALIGN
    assert g(None, 64, None, None, None, 64, 0, 64, 64, 0, None, 0, None) == OK
    assert g(None, 64, None, None, None, 64, 64, 0, 64, 0, None, 0, None) == OK
    # the workspace must be 256-byte aligned (16-byte aligned is not enough)
    W16 = P((1 << 20) + 16)
    assert g(A, 64, B, C, D, 64, 64, 64, 64, 0, W16, ws, None) == ALIGN
    # the no-allocation variant: same rules, no workspace; shapes beyond its scratch are refused
    z = L.bsq_gemm_fp8r_noalloc
    with open(os.path.join(ROOT, "include", "bsq.h")) as f:
        assert "#define BSQ_NOALLOC_MAX_BYTES ((size_t)64 << 20)" in f.read()
    assert z(A, 64, B, None, D, 64, 64, 64, 64, 0, None) == NULL
    assert z(A, 64, B, C, D, 64, 64, 64, 48, 0, None) == SHAPE
    assert z(A, 64, B, C, D, 64, 64, 64, 64, 2, None) == ARG
    assert z(None, 64, None, None, None, 64, 0, 64, 64, 0, None) == OK
    big_m = _lib.BSQ_NOALLOC_MAX_BYTES // 4096 + 1                                      # M * K just over 64 MiB
    assert z(A, 4096, B, C, D, 64, big_m, 64, 4096, 0, None) == WS
    n = L.bsq_gemm_nvfp4
    assert n(A, 64, B, C, D, D, A, 64, 64, 64, 64, 0, W16, 1 << 20, None) == ALIGN
    assert n(A, 64, B, C, D, None, A, 64, 64, 64, 64, 0, A, 1 << 20, None) == NULL       # W4A4 needs input_scale
    assert n(A, 64, B, C, None, D, A, 64, 64, 64, 64, 0, A, 1 << 20, None) == NULL       # w_scale2
    assert n(A, 64, B, C, D, D, A, 64, 64, 64, 64, 0, None, 0, None) == WS
    assert n(A, 64, B, ODD, D, D, A, 64, 64, 64, 64, 0, A, 1 << 20, None) == ALIGN
    assert n(A, 64, B, C, D, None, A, 64, 64, 64, 64, 4, None, 0, None) == ARG


def test_quantize_y_validation():
    q = L.bsq_gemm_nvfp4_q_quantize_y
    # xq, x_bscale, input_scale, w, w_bscale, w_scale2, y_scale, yq, y_bscale, y, ldy, M, N, K, ws, ws_bytes, stream
    assert q(A, B, C, A, B, C, D, A, B, None, 0, 64, 48, 256, None, 0, None) == SHAPE     # N % 32
    assert q(A, B, C, A, B, C, D, A, B, D, 68, 64, 64, 256, None, 0, None) == SHAPE       # ldy % 8
    assert q(A, B, C, A, B, C, None, A, B, None, 0, 64, 64, 256, None, 0, None) == NULL   # y_scale
    assert q(A, B, C, A, B, C, D, A, None, None, 0, 64, 64, 256, None, 0, None) == NULL   # y_bscale
    assert q(A, B, C, A, B, C, D, ODD, B, None, 0, 64, 64, 256, None, 0, None) == ALIGN  # yq
    assert q(A, B, C, A, B, C, D, A, B, None, 0, 0, 64, 256, None, 0, None) == OK         # empty
    # K % 256 != 0 beyond the few-token range has no fused kernel: without y it needs a workspace
    assert L.bsq_gemm_nvfp4_quantize_y_workspace_bytes(4096, 1024, 96, 0) == 4096 * 1024 * 2
    assert L.bsq_gemm_nvfp4_quantize_y_workspace_bytes(4096, 1024, 96, 1) == 0
    assert L.bsq_gemm_nvfp4_quantize_y_workspace_bytes(4096, 1024, 512, 0) == 0
    assert L.bsq_gemm_nvfp4_quantize_y_workspace_bytes(16, 1024, 96, 0) == 0
    assert q(A, B, C, A, B, C, D, A, B, None, 0, 4096, 1024, 96, None, 0, None) == WS


def test_quantized_output_validation():
    fp8, nv = _lib.BSQ_FMT_FP8R, _lib.BSQ_FMT_NVFP4
    pad = lambda n: (n + 255) // 256 * 256
    wsb = L.bsq_gemm_quantize_y_workspace_bytes
    assert wsb(fp8, 4096, 3072, 1) == pad(48 * 4096 * 4)                    # row maxima per 64 columns
    assert wsb(fp8, 4096, 3072, 0) == pad(4096 * 3072 * 2) + pad(48 * 4096 * 4)
    assert wsb(nv, 4096, 3072, 1) == 0 and wsb(nv, 4096, 3072, 0) == pad(4096 * 3072 * 2)
    assert wsb(fp8, 0, 3072, 0) == 0 and wsb(3, 64, 64, 0) == 0
    g = L.bsq_gemm_fp8r_q_quantize_y
    ws = wsb(fp8, 64, 64, 0)
    # xq, x_scale, w, w_scale, out_fmt, y_global, yq, yq_scale, y, ldy, M, N, K, ws, ws_bytes, stream
    assert g(A, B, C, D, 3, None, A, B, None, 0, 64, 64, 64, A, ws, None) == ARG          # format
    assert g(A, B, C, D, fp8, D, A, B, None, 0, 64, 64, 64, A, ws, None) == ARG           # fp8r takes no global
    assert g(A, B, C, D, nv, None, A, B, None, 0, 64, 64, 64, A, ws, None) == NULL         # nvfp4 needs one
    assert g(A, B, C, D, fp8, None, A, B, None, 0, 64, 48, 64, A, ws, None) == SHAPE       # N % 32
    assert g(A, B, C, D, fp8, None, ODD, B, None, 0, 64, 64, 64, A, ws, None) == ALIGN     # yq
    assert g(A, B, C, D, fp8, None, A, B, None, 0, 64, 64, 64, A, ws - 1, None) == WS
    assert g(A, B, C, D, fp8, None, A, B, None, 0, 64, 64, 64, P((1 << 20) + 16), ws, None) == ALIGN
    assert g(A, None, C, D, fp8, None, A, B, None, 0, 64, 64, 64, A, ws, None) == NULL     # x_scale
    assert g(None, None, None, None, fp8, None, None, None, None, 0, 0, 64, 64, None, 0, None) == OK  # empty
    n = L.bsq_gemm_nvfp4_q_quantize_y_fp8r
    # xq, x_bscale, input_scale, w, w_bscale, w_scale2, yq, y_rowscale, y, ldy, M, N, K, ws, ws_bytes, stream
    assert n(A, B, None, A, B, C, A, B, None, 0, 64, 64, 256, A, ws, None) == NULL         # input_scale
    assert n(A, B, C, A, B, C, A, None, None, 0, 64, 64, 256, A, ws, None) == NULL         # row scales
    assert n(A, B, C, A, B, C, A, B, None, 0, 64, 64, 256, None, 0, None) == WS
    assert n(A, B, C, A, B, C, A, B, D, 68, 64, 64, 256, A, ws, None) == SHAPE             # ldy % 8
    assert n(None, None, None, None, None, None, None, None, None, 0, 0, 64, 256, None, 0, None) == OK


def test_lora_validation():
    pad = lambda n: (n + 255) // 256 * 256
    fp8, nv, wo = _lib.BSQ_FMT_FP8R, _lib.BSQ_FMT_NVFP4, _lib.BSQ_WEIGHT_ONLY
    wsb = L.bsq_lora_workspace_bytes
    # the linear's workspace, T, and the fp32 partials of the K slices: at 4096 tokens K = 3072
    # is cut into 12 slices of 256 for rank 32 (384 workgroups), 3 of 1024 for rank 128 (partials
    # within a quarter of X's bytes)
    assert L.bsq_lora_down_workspace_bytes(4096, 3072, 32) == pad(12 * 4096 * 32 * 4)
    assert L.bsq_lora_down_workspace_bytes(4096, 3072, 128) == pad(3 * 4096 * 128 * 4)
    assert wsb(fp8, 4096, 3072, 3072, 32, 0) == (L.bsq_gemm_workspace_bytes(fp8, 4096, 3072, 3072, 0) + pad(4096 * 64)
                                                 + pad(12 * 4096 * 32 * 4))
    assert wsb(nv, 4096, 12288, 3072, 16, wo) == pad(4096 * 32) + pad(12 * 4096 * 16 * 4)
    # many row blocks: one slice, no partials
    assert L.bsq_lora_down_workspace_bytes(65536, 3072, 32) == 0
    assert wsb(nv, 0, 12288, 3072, 16, 0) == 0 and wsb(3, 64, 64, 64, 16, 0) == 0
    g = L.bsq_gemm_fp8r_lora
    ws = wsb(fp8, 64, 64, 64, 16, 0)
    # x, ldx, w, w_scale, a, b, rank, scale, y, ldy, M, N, K, flags, ws, ws_bytes, stream
    assert g(A, 64, B, C, A, B, 16, 1.0, D, 64, 64, 64, 64, 0, A, ws - 1, None) == WS
    assert g(A, 64, B, C, A, B, 0, 1.0, D, 64, 64, 64, 64, 0, A, ws, None) == SHAPE       # rank 0
    assert g(A, 64, B, C, A, B, 129, 1.0, D, 64, 64, 64, 64, 0, A, 1 << 24, None) == SHAPE  # rank > 128
    assert g(A, 64, B, C, A, B, 16, float("nan"), D, 64, 64, 64, 64, 0, A, ws, None) == ARG
    assert g(A, 64, B, C, A, B, 16, float("inf"), D, 64, 64, 64, 64, 0, A, ws, None) == ARG
    assert g(A, 64, B, C, None, B, 16, 1.0, D, 64, 64, 64, 64, 0, A, ws, None) == NULL
    assert g(A, 64, B, C, A, ODD, 16, 1.0, D, 64, 64, 64, 64, 0, A, ws, None) == ALIGN
    assert g(A, 1 << 24, B, C, A, B, 16, 1.0, D, 64, 4, 64, 64, 0, A, 1 << 30, None) == SHAPE  # ldx
    assert g(A, 64, B, C, A, B, 128, 1.0, D, 1 << 22, 1 << 22, 64, 64, 0, A, 1 << 40, None) == SHAPE  # M * rank
    assert g(None, 64, None, None, A, B, 16, 1.0, None, 64, 0, 64, 64, 0, None, 0, None) == OK  # empty
    # an empty call touches no pointer, the adapter's included
    assert g(None, 64, None, None, None, None, 16, 1.0, None, 64, 0, 64, 64, 0, None, 0, None) == OK
    assert g(None, 64, None, None, None, None, 16, 1.0, None, 64, 64, 0, 64, 0, None, 0, None) == OK
    n = L.bsq_gemm_nvfp4_lora
    ws = wsb(nv, 64, 64, 64, 16, 0)
    # x, ldx, w, w_bscale, w_scale2, input_scale, a, b, rank, scale, y, ldy, M, N, K, flags, ws, ws_bytes, stream
    assert n(A, 64, B, C, D, None, A, B, 16, 1.0, D, 64, 64, 64, 64, 0, A, ws, None) == NULL     # input_scale
    assert n(A, 64, B, C, D, D, A, B, 16, 1.0, D, 64, 64, 64, 64, 0, A, ws - 1, None) == WS
    assert n(A, 64, B, C, D, None, A, B, 16, 1.0, D, 64, 64, 64, 64, wo, None, 0, None) == WS    # T needs room
    assert n(A, 64, B, C, D, D, A, B, 16, 1.0, D, 64, 64, 64, 64, 8, A, ws, None) == ARG
    assert n(None, 64, None, None, None, None, None, None, 16, 1.0, None, 64, 0, 64, 64, 0, None, 0, None) == OK
    d = L.bsq_lora_down
    # x, ldx, a, M, K, rank, scale, t, ws, ws_bytes, stream
    assert d(A, 64, B, 4, 64, 0, 1.0, C, None, 0, None) == SHAPE
    assert d(A, 64, B, 4, 48, 16, 1.0, C, None, 0, None) == SHAPE                 # K % 32
    assert d(A, 64, B, 4, 64, 16, float("nan"), C, None, 0, None) == ARG
    assert d(A, 64, None, 4, 64, 16, 1.0, C, None, 0, None) == NULL
    assert d(A, 64, B, 4, 64, 16, 1.0, ODD, None, 0, None) == ALIGN
    assert d(A, 3072, B, 4, 3072, 16, 1.0, C, None, 0, None) == WS                # K is split: partials
    assert d(None, 64, None, 0, 64, 16, 1.0, None, None, 0, None) == OK


def test_dequant_validation():
    d = L.bsq_dequant_to_bf16
    assert d(3, A, B, C, 4, 64, D, None) == ARG
    assert d(_lib.BSQ_FMT_FP8R, A, B, C, 4, 64, D, None) == ARG      # fp8r takes no global scale
    assert d(_lib.BSQ_FMT_NVFP4, A, B, None, 4, 64, D, None) == NULL
    assert d(_lib.BSQ_FMT_NVFP4, A, B, C, 4, 40, D, None) == SHAPE
    assert d(_lib.BSQ_FMT_NVFP4, A, B, C, 4, 64, ODD, None) == ALIGN
    assert d(_lib.BSQ_FMT_FP8R, None, None, None, 0, 64, None, None) == OK


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="only meaningful without a GPU")
def test_valid_call_without_gpu_reports_device_error():
    assert L.bsq_quantize_act_fp8r(A, 4, 64, 64, B, C, None) == DEV
    assert L.bsq_dequant_to_bf16(_lib.BSQ_FMT_FP8R, A, B, None, 4, 64, D, None) == DEV


def test_binding_checks_tensors_before_calling():
    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        _lib.bsq_quantize_act_fp8r(x)          # CPU tensor is rejected by the binding


def test_binding_counts_workspace_bytes_of_any_dtype():
    # a caller's workspace of another dtype is passed with its size in bytes, not elements
    assert _lib._nbytes(torch.empty(10, dtype=torch.float32)) == 40
    assert _lib._nbytes(torch.empty(10, dtype=torch.uint8)) == 10
    assert _lib._nbytes(None) == 0
