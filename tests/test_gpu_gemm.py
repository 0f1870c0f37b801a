"""GPU parity: fp8r and nvfp4 GEMMs against the oracle's fp64 products.

Weights are quantized by the oracle from seeded bf16 tensors and uploaded;
activations go up as bf16 and are quantized inside the GEMM entry points (the
GPU quantizers are checked bit-exact separately), so Y is compared with the
oracle's exact product of the dequantized operands under the stated
tolerance. Large shapes are compared on sampled rows.
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_row_amd import synthetic as syn
from oracle import codec, gemm, quant
from tests.gpu_util import assert_gemm_close, assert_gemm_close_by_row, dev, dev_bf16, dev_scalar, host

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from block_scaled_precision_row_amd import _lib as L


def _rows_subset(M, n, seed):
    if M <= n:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, M - 1], rng.choice(M, n - 2, replace=False)]))


def run_fp8r(x, w, weight_only=False, sample=None, what=""):
    M, K = x.shape
    wq, sw = quant.quantize_fp8r(w)
    flags = L.BSQ_WEIGHT_ONLY if weight_only else 0
    y = L.bsq_gemm_fp8r(dev_bf16(x), dev(wq), dev(sw), flags=flags)
    torch.cuda.synchronize()
    yb = host(y)
    rows = _rows_subset(M, sample, M) if sample else np.arange(M)
    if weight_only:
        ref = gemm.gemm_fp8r_weight_only(x[rows], wq, sw)
    else:
        xq, sx = quant.quantize_fp8r(x[rows])
        ref = gemm.gemm_fp8r(xq, sx, wq, sw)
    assert_gemm_close(yb[rows], ref, what)
    return yb


def run_nvfp4(x, w, weight_only=False, sample=None, what=""):
    M, K = x.shape
    gw = quant.calibrate_global_scale(w)
    wq, sfw = quant.quantize_nvfp4(w, gw)
    gx = quant.calibrate_global_scale(x)
    flags = L.BSQ_WEIGHT_ONLY if weight_only else 0
    y = L.bsq_gemm_nvfp4(dev_bf16(x), dev(wq), dev(sfw), dev_scalar(gw),
                         None if weight_only else dev_scalar(gx), flags=flags)
    torch.cuda.synchronize()
    yb = host(y)
    rows = _rows_subset(M, sample, M + 1) if sample else np.arange(M)
    if weight_only:
        ref = gemm.gemm_nvfp4_weight_only(x[rows], wq, sfw, gw)
    else:
        xq, sfx = quant.quantize_nvfp4(x[rows], gx)
        ref = gemm.gemm_nvfp4(xq, sfx, gx, wq, sfw, gw)
    assert_gemm_close(yb[rows], ref, what)
    return yb


SMALL_SHAPES = [(64, 128, 256), (77, 100, 96), (1, 8, 32), (130, 257, 160), (256, 192, 512), (300, 520, 1056)]


@pytest.mark.parametrize("M,N,K", SMALL_SHAPES)
def test_fp8r_small_and_ragged(M, N, K):
    x = syn.normal_bf16((M, K), 50, M, outlier_frac=0.01)
    w = syn.normal_bf16((N, K), 50, 1000 + N, sigma=0.02)
    run_fp8r(x, w, what="fp8r %dx%dx%d" % (M, N, K))
    run_fp8r(x, w, weight_only=True, what="fp8r-w8a16 %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", SMALL_SHAPES)
def test_nvfp4_small_and_ragged(M, N, K):
    x = syn.normal_bf16((M, K), 51, M)
    w = syn.normal_bf16((N, K), 51, 1000 + N, sigma=0.02)
    run_nvfp4(x, w, what="nvfp4-w4a4 %dx%dx%d" % (M, N, K))
    run_nvfp4(x, w, weight_only=True, what="nvfp4-w4a16 %dx%dx%d" % (M, N, K))


def test_tiny_weight_only_workload():
    """64x256 activations, 128x256 nvfp4 weights, weight-only: the smallest workload."""
    x = syn.activations(syn.TINY, 64, 256)
    w = syn.weights(syn.TINY, 128, 256)
    run_nvfp4(x, w, weight_only=True, what="tiny w4a16")


def test_fp8r_w8a8_4096x3072x3072():
    x = syn.activations(syn.FP8R_4096, 4096, 3072)
    w = syn.weights(syn.FP8R_4096, 3072, 3072)
    y1 = run_fp8r(x, w, what="fp8r 4096x3072x3072")
    y2 = host(L.bsq_gemm_fp8r(dev_bf16(x), *[dev(t) for t in quant.quantize_fp8r(w)]))
    torch.cuda.synchronize()
    assert np.array_equal(y1, y2), "not deterministic"


def test_nvfp4_w4a4_mlp_up_4096x12288x3072():
    x = syn.activations(syn.NVFP4_UP, 4096, 3072)
    w = syn.weights(syn.NVFP4_UP, 12288, 3072)
    run_nvfp4(x, w, sample=512, what="nvfp4 4096x12288x3072")


@pytest.mark.parametrize("N", [3072, 12288])
def test_small_m_512(N):
    x = syn.activations(syn.SMALL_M, 512, 3072)
    w = syn.weights(syn.SMALL_M, N, 3072, tensor_id=syn.W_ID if N == 3072 else syn.W2_ID)
    run_nvfp4(x, w, what="small-M w4a4 N=%d" % N)
    run_nvfp4(x, w, weight_only=True, what="small-M w4a16 N=%d" % N)
    run_fp8r(x, w, what="small-M w8a8 N=%d" % N)


@pytest.mark.parametrize("gi,block", [(0, 0), (1, 1), (3, 2), (2, 3)])
def test_joint_block_4mp_sampled(gi, block):
    """Joint-block GEMMs at 16384 tokens, compared on 64 sampled rows."""
    name, N, K = syn.JOINT_GEMMS[gi]
    x = syn.activations(syn.JOINT_4MP, syn.JOINT_TOKENS, K, block=0 if K == 3072 else 1)
    w = syn.weights(syn.JOINT_4MP, N, K, block=block * 4 + gi)
    if syn.joint_scheme(block) == "nvfp4":
        run_nvfp4(x, w, sample=64, what="joint %s block %d nvfp4" % (name, block))
    else:
        run_fp8r(x, w, sample=64, what="joint %s block %d fp8r" % (name, block))


def test_weight_only_differs_slightly_from_fused():
    x = syn.activations(syn.SMALL_M, 256, 3072)
    w = syn.weights(syn.SMALL_M, 512, 3072)
    a = run_nvfp4(x, w, what="w4a4")
    b = run_nvfp4(x, w, weight_only=True, what="w4a16")
    fa, fb = [(t.astype(np.uint32) << 16).view(np.float32).astype(np.float64) for t in (a, b)]
    rel = np.linalg.norm(fa - fb) / np.linalg.norm(fb)
    assert 0.005 < rel < 0.3


def test_empty_m_is_a_noop():
    w = syn.weights(syn.TINY, 64, 256)
    wq, sw = quant.quantize_fp8r(w)
    y = L.bsq_gemm_fp8r(torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"), dev(wq), dev(sw))
    assert tuple(y.shape) == (0, 64)


def test_strided_activations_and_output():
    M, N, K = 96, 136, 256
    x = syn.normal_bf16((M, K), 52, 1)
    w = syn.normal_bf16((N, K), 52, 2, sigma=0.02)
    xp = np.zeros((M, K + 40), np.uint16)
    xp[:, :K] = x
    xd = dev_bf16(xp)[:, :K]
    ybig = torch.zeros((M, N + 6), dtype=torch.bfloat16, device="cuda")
    y = ybig[:, :N]
    wq, sw = quant.quantize_fp8r(w)
    L.bsq_gemm_fp8r(xd, dev(wq), dev(sw), y=y)
    gw = quant.calibrate_global_scale(w)
    p, s = quant.quantize_nvfp4(w, gw)
    ybig2 = torch.zeros((M, N + 6), dtype=torch.bfloat16, device="cuda")
    L.bsq_gemm_nvfp4(xd, dev(p), dev(s), dev_scalar(gw), flags=L.BSQ_WEIGHT_ONLY, y=ybig2[:, :N])
    torch.cuda.synchronize()
    xq, sx = quant.quantize_fp8r(x)
    assert_gemm_close(host(ybig)[:, :N], gemm.gemm_fp8r(xq, sx, wq, sw), "strided fp8r")
    assert np.all(host(ybig)[:, N:] == 0)
    assert_gemm_close(host(ybig2)[:, :N], gemm.gemm_nvfp4_weight_only(x, p, s, gw), "strided w4a16")
    assert np.all(host(ybig2)[:, N:] == 0)


@pytest.mark.parametrize("M,N,K", [(4096, 12288, 3072), (77, 100, 96), (300, 520, 1056), (256, 256, 512)])
def test_prequantized_activation_entry_points(M, N, K):
    """GEMMs on oracle-quantized activations: the same bytes on both sides, so only the GEMM is under test."""
    x = syn.normal_bf16((M, K), 53, M)
    w = syn.normal_bf16((N, K), 53, N, sigma=0.02)
    rows = _rows_subset(M, 256, 7)
    gx, gw = quant.calibrate_global_scale(x), quant.calibrate_global_scale(w)
    xq, sfx = quant.quantize_nvfp4(x, gx)
    wq, sfw = quant.quantize_nvfp4(w, gw)
    y = L.bsq_gemm_nvfp4_q(dev(xq), dev(sfx), dev_scalar(gx), dev(wq), dev(sfw), dev_scalar(gw))
    x8, s8 = quant.quantize_fp8r(x)
    w8, t8 = quant.quantize_fp8r(w)
    y8 = L.bsq_gemm_fp8r_q(dev(x8), dev(s8), dev(w8), dev(t8))
    torch.cuda.synchronize()
    assert_gemm_close(host(y)[rows], gemm.gemm_nvfp4(xq[rows], sfx[rows], gx, wq, sfw, gw), "nvfp4_q %dx%dx%d" % (M, N, K))
    assert_gemm_close(host(y8)[rows], gemm.gemm_fp8r(x8[rows], s8[rows], w8, t8), "fp8r_q %dx%dx%d" % (M, N, K))


# Few tokens: these shapes run on the skinny kernel (K split over the waves of a workgroup);
# K values chosen so that stages end inside a lane's window (544 = 4 * 128 + 32) and waves
# without any stage exist (K = 96, 224). Wave counts per workgroup other than the default:
# 40 x 8200 x 544 runs the four-wave W4A4 and W4A16 variants (>= 256 workgroups), 3 x 8200 x
# 1056 and 5 x 12288 x 3072 the two-wave W8A16 one (>= 256 workgroups, <= 16 tokens), 7 x 700 x
# 544 the eight-wave W8A8 one (<= 8 tokens, small grid), all with ragged weight blocks.
SKINNY_SHAPES = [(16, 3072, 3072), (33, 1000, 544), (64, 3072, 3072), (96, 520, 224), (160, 3072, 3072),
                 (256, 1056, 96), (5, 12288, 3072), (40, 8200, 544), (3, 8200, 1056), (7, 700, 544)]


@pytest.mark.parametrize("M,N,K", SKINNY_SHAPES)
def test_skinny_all_schemes(M, N, K):
    x = syn.normal_bf16((M, K), 52, M, outlier_frac=0.01)
    w = syn.normal_bf16((N, K), 52, 2000 + N + K, sigma=0.02)
    tag = "%dx%dx%d" % (M, N, K)
    run_fp8r(x, w, what="fp8r " + tag)
    run_fp8r(x, w, weight_only=True, what="fp8r-w8a16 " + tag)
    run_nvfp4(x, w, what="nvfp4 " + tag)
    run_nvfp4(x, w, weight_only=True, what="nvfp4-w4a16 " + tag)


# W4A4 shapes with more output tiles than compute units, ragged M and N tails, the 256 x 192
# tile over two rounds and over one, the 128 x 128 tile (1000 x 5000), and both parities of
# the number of 256-deep K stages per tile.
PERSISTENT_SHAPES = [(4100, 4100, 768), (4100, 4100, 1024), (1000, 5000, 512), (4100, 2300, 1024)]


@pytest.mark.parametrize("M,N,K", PERSISTENT_SHAPES)
def test_w4a4_several_tiles_per_workgroup(M, N, K):
    x = syn.normal_bf16((M, K), 53, M)
    w = syn.normal_bf16((N, K), 53, 3000 + N, sigma=0.02)
    run_nvfp4(x, w, sample=96, what="nvfp4 rounds %dx%dx%d" % (M, N, K))


# fp8r grids whose 256 x 256 tiles fill whole rounds on the compute units no worse than the
# other tiles' run the square tile: ragged M and N tails, K of several 128-deep stages and one
# with a half stage (K % 128 == 64). 6100 x 5400 runs 256 x 192 tiles over three rounds.
SQUARE_FP8_SHAPES = [(6100, 5400, 512), (8192, 4096, 320), (16384, 9216, 256)]


@pytest.mark.parametrize("M,N,K", SQUARE_FP8_SHAPES)
def test_fp8r_square_tiles(M, N, K):
    x = syn.normal_bf16((M, K), 56, M, outlier_frac=0.01)
    w = syn.normal_bf16((N, K), 56, 6000 + N, sigma=0.02)
    run_fp8r(x, w, sample=96, what="fp8r square tiles %dx%dx%d" % (M, N, K))


# The large-grid tile choice counts whole rounds of tiles on the 256 compute units: 3100 x
# 4000 takes 256 x 256 tiles in one round (256 x 192 would need two), 4100 x 4100 takes 256 x
# 192 tiles in two rounds (256 x 256 and 128 x 128 would need two and five), 1000 x 5000 takes
# 128 x 128 tiles (on the fp8r GEMM two workgroups a compute unit), on both the fp8r and the W4A4
# GEMM; all with ragged M and N tails.
ROUND_SHAPES = [(3100, 4000, 768), (4100, 4100, 768), (1000, 5000, 512)]


@pytest.mark.parametrize("M,N,K", ROUND_SHAPES)
def test_large_grid_tile_choice(M, N, K):
    x = syn.normal_bf16((M, K), 57, M + N, outlier_frac=0.01)
    w = syn.normal_bf16((N, K), 57, 7000 + N, sigma=0.02)
    run_fp8r(x, w, sample=96, what="fp8r rounds %dx%dx%d" % (M, N, K))
    run_nvfp4(x, w, sample=96, what="nvfp4 rounds %dx%dx%d" % (M, N, K))


# Between 256 and 512 tiles of 128 x 128 (K % 128 == 0) the fp8r GEMM runs them two workgroups
# a compute unit on the hand-ordered loop: 2048 x 3072 (384 tiles), ragged 2500 x 3000 (480) and
# 1500 x 3000 (288, K = 384: three stages); the same bits as any other tile.
PAIR_SHAPES = [(2048, 3072, 3072), (2500, 3000, 512), (1500, 3000, 384)]


@pytest.mark.parametrize("M,N,K", PAIR_SHAPES)
def test_fp8r_paired_tiles(M, N, K):
    x = syn.normal_bf16((M, K), 58, M + N, outlier_frac=0.01)
    w = syn.normal_bf16((N, K), 58, 7500 + N, sigma=0.02)
    run_fp8r(x, w, sample=96, what="fp8r paired 128x128 %dx%dx%d" % (M, N, K))


# Small grids (a few hundred tokens) run 64 x 64 or 64 x 128 tiles: ragged M and N tails, two
# workgroups' worth of tokens, one 64-token block with the ragged 65th row, and the 512-token
# weight-streaming shape
SMALL_GRID_SHAPES = [(300, 520, 1024), (65, 12288, 512), (200, 3000, 768), (512, 3072, 3072)]


@pytest.mark.parametrize("M,N,K", SMALL_GRID_SHAPES)
def test_small_grid_tiles(M, N, K):
    x = syn.normal_bf16((M, K), 60, M + N, outlier_frac=0.01)
    w = syn.normal_bf16((N, K), 60, 8000 + N, sigma=0.02)
    big = M * N > 1 << 20
    run_fp8r(x, w, sample=64 if big else None, what="fp8r small grid %dx%dx%d" % (M, N, K))
    run_nvfp4(x, w, sample=64 if big else None, what="nvfp4 small grid %dx%dx%d" % (M, N, K))


# Weight-only (W4A16, W8A16) tiled kernel, tiles chosen by whole rounds on the compute units:
# nvfp4 256 x 128 (2000 x 3000, 2000 x 4000), 256 x 192 (4096 x 3072, 3000 x 3000), E4M3
# 128 x 192 (2000 x 3000, 4096 x 3072, 3000 x 3000), 128 x 256 (2000 x 4000), both 128 x 128
# (1000 x 4000) and the small-grid tiles, with ragged M and N, and a K whose last 128-deep
# stage is half full (the nvfp4 block-scale copies of its second half read as zeros)
A16_SHAPES = [(2000, 3000, 1024), (300, 700, 2112), (4096, 3072, 3072), (2000, 4000, 1024), (3000, 3000, 1088),
              (1000, 4000, 1024),
              (300, 200, 64), (257, 136, 32)]  # K below one 128-deep stage (K = 32: W8A16 only here)


@pytest.mark.parametrize("M,N,K", A16_SHAPES)
def test_weight_only_tiled(M, N, K):
    x = syn.normal_bf16((M, K), 61, M + N)
    w = syn.normal_bf16((N, K), 61, 9000 + N, sigma=0.02)
    sample = 64 if M * N > 1 << 20 else None
    run_fp8r(x, w, weight_only=True, sample=sample, what="w8a16 %dx%dx%d" % (M, N, K))
    run_nvfp4(x, w, weight_only=True, sample=sample, what="w4a16 %dx%dx%d" % (M, N, K))


# ---- edge inputs through the GEMM entry points ----------------------------------------------
# The quantizers' edge rows (zero rows, signed zeros, zero blocks, row magnitudes spread over
# 2^-40 .. 2^40) fed to whole linears, on shapes that take the few-token, small-grid and tiled
# kernels; each row is held to the tolerance on its own.
EDGE_SHAPES = [(16, 384, 512), (96, 320, 512), (600, 1024, 1024)]


def _edge_rows(M, K, seed):
    from tests.test_gpu_quant import _varied_rows
    return _varied_rows(M, K, seed)


@pytest.mark.parametrize("M,N,K", EDGE_SHAPES)
def test_fp8r_edge_rows(M, N, K):
    x = _edge_rows(M, K, 60 + M)
    w = syn.normal_bf16((N, K), 60, 1000 + N, sigma=0.02)
    wq, sw = quant.quantize_fp8r(w)
    y = host(L.bsq_gemm_fp8r(dev_bf16(x), dev(wq), dev(sw)))
    xq, sx = quant.quantize_fp8r(x)
    assert_gemm_close_by_row(y, gemm.gemm_fp8r(xq, sx, wq, sw), "fp8r edge rows %dx%dx%d" % (M, N, K))
    y = host(L.bsq_gemm_fp8r(dev_bf16(x), dev(wq), dev(sw), flags=L.BSQ_WEIGHT_ONLY))
    assert_gemm_close_by_row(y, gemm.gemm_fp8r_weight_only(x, wq, sw), "fp8r-w8a16 edge rows %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", EDGE_SHAPES)
def test_nvfp4_edge_rows(M, N, K):
    """W4A4 with the global scale calibrated on the whole X: rows far below the largest ones
    quantize to zero blocks (scale code 0), as the oracle's do."""
    x = _edge_rows(M, K, 70 + M)
    w = syn.normal_bf16((N, K), 70, 1000 + N, sigma=0.02)
    gw = quant.calibrate_global_scale(w)
    wq, sfw = quant.quantize_nvfp4(w, gw)
    gx = quant.calibrate_global_scale(x)
    y = host(L.bsq_gemm_nvfp4(dev_bf16(x), dev(wq), dev(sfw), dev_scalar(gw), dev_scalar(gx)))
    xq, sfx = quant.quantize_nvfp4(x, gx)
    assert_gemm_close_by_row(y, gemm.gemm_nvfp4(xq, sfx, gx, wq, sfw, gw), "nvfp4 edge rows %dx%dx%d" % (M, N, K))
    y = host(L.bsq_gemm_nvfp4(dev_bf16(x), dev(wq), dev(sfw), dev_scalar(gw), None, flags=L.BSQ_WEIGHT_ONLY))
    assert_gemm_close_by_row(y, gemm.gemm_nvfp4_weight_only(x, wq, sfw, gw),
                             "nvfp4-w4a16 edge rows %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [(16, 384, 512), (300, 520, 1056), (1024, 1536, 3072)])
def test_w4a4_saturating_input_scale(M, N, K):
    """An input_scale 64x below the data's calibrated one: block scales saturate at 448 and
    codes at +-6 inside the linear, exactly as the oracle's quantizer saturates them."""
    x = syn.normal_bf16((M, K), 80, M)
    w = syn.normal_bf16((N, K), 80, 1000 + N, sigma=0.02)
    gw = quant.calibrate_global_scale(w)
    wq, sfw = quant.quantize_nvfp4(w, gw)
    gx = np.float32(quant.calibrate_global_scale(x) / 64)
    xq, sfx = quant.quantize_nvfp4(x, gx)
    assert (sfx == 0x7E).mean() > 0.5          # most blocks saturate
    y = host(L.bsq_gemm_nvfp4(dev_bf16(x), dev(wq), dev(sfw), dev_scalar(gw), dev_scalar(gx)))
    assert_gemm_close(y, gemm.gemm_nvfp4(xq, sfx, gx, wq, sfw, gw), "w4a4 saturating %dx%dx%d" % (M, N, K))
