"""GPU parity of the LoRA side path: y = linear(x) + s (x A^T) B^T on every GEMM route.

The oracle's output is the fp64 base product (as in test_gpu_gemm.py) plus the
adapter's exact fp64 contribution. The GPU rounds the output once, as the
GEMMs do, and also holds the rank-r intermediate T in bf16; the comparison is
the GEMM tolerance plus that rounding's elementwise bound (the adapter term is
10-30 % of the output here, so a dropped scale, term or transpose fails it).
With a zero scale the LoRA entry points must reproduce the plain entry points
bit for bit on every route. Shapes are picked to reach every kernel: few-token
(skinny) kernels, the 128 x 128 and 256 x 256 / 256 x 192 tiled kernels, the
decode-GEMM fallback (K % 256 != 0), ragged M / N tails, and ranks that are
not multiples of 8 or 16.
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_row_amd import synthetic as syn
from oracle import codec, gemm, lora, quant
from tests.gpu_util import assert_gemm_close, dev, dev_bf16, dev_scalar, host

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from block_scaled_precision_row_amd import _lib as L

SCALE = 0.75  # not 1, so that an ignored scale shows


def _rows_subset(M, n, seed):
    if M <= n:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, M - 1], rng.choice(M, n - 2, replace=False)]))


def _inputs(M, N, K, rank, wid):
    x = syn.normal_bf16((M, K), 60, M + 7 * K)
    w = syn.normal_bf16((N, K), 60, 5000 + N + K, sigma=0.02)
    a, b = syn.lora_adapter(60, rank, N, K, block=wid)
    return x, w, a, b


def run_lora(scheme, weight_only, x, w, a, b, scale, sample=None, what=""):
    M, K = x.shape
    flags = L.BSQ_WEIGHT_ONLY if weight_only else 0
    rows = _rows_subset(M, sample, M + 3) if sample else np.arange(M)
    da, db = dev_bf16(a), dev_bf16(b)
    if scheme == "fp8r":
        wq, sw = quant.quantize_fp8r(w)
        y = L.bsq_gemm_fp8r_lora(dev_bf16(x), dev(wq), dev(sw), da, db, scale, flags=flags)
        torch.cuda.synchronize()
        if weight_only:
            base = gemm.gemm_fp8r_weight_only(x[rows], wq, sw)
        else:
            xq, sx = quant.quantize_fp8r(x[rows])
            base = gemm.gemm_fp8r(xq, sx, wq, sw)
    else:
        gw = quant.calibrate_global_scale(w)
        wq, sfw = quant.quantize_nvfp4(w, gw)
        gx = quant.calibrate_global_scale(x)
        y = L.bsq_gemm_nvfp4_lora(dev_bf16(x), dev(wq), dev(sfw), dev_scalar(gw),
                                  None if weight_only else dev_scalar(gx), da, db, scale, flags=flags)
        torch.cuda.synchronize()
        if weight_only:
            base = gemm.gemm_nvfp4_weight_only(x[rows], wq, sfw, gw)
        else:
            xq, sfx = quant.quantize_nvfp4(x[rows], gx)
            base = gemm.gemm_nvfp4(xq, sfx, gx, wq, sfw, gw)
    ref = lora.lora_linear(base, x[rows], a, b, scale)
    delta = ref - base
    share = np.linalg.norm(delta) / max(np.linalg.norm(ref), 1e-300)
    assert_gemm_close(host(y)[rows], ref, "%s adapter share %.2f" % (what, share),
                      extra=t_rounding_bound(x[rows], a, b, scale))
    return y


def t_rounding_bound(x, a, b, scale):
    """Elementwise bound of what holding T = s X A^T in bf16 changes in T B^T: each T value
    moves by at most 2^-9 of itself (round to nearest), plus fp32 accumulation slack, so the
    product moves by at most 2^-9 sum_j |T[m][j]| |B[n][j]|; twice that is allowed."""
    t = np.abs(lora.lora_down(x, a, scale))
    return 2.0 ** -8 * (t @ np.abs(codec.bf16_to_f64(b)).T)


SCHEMES = [("fp8r", False), ("fp8r", True), ("nvfp4", False), ("nvfp4", True)]

# (M, N, K, rank)
ROUTE_SHAPES = [
    (1, 64, 256, 5),        # few-token kernels, odd rank (two-byte adapter loads)
    (20, 1024, 512, 32),    # few-token kernels
    (100, 300, 96, 8),      # few-token kernels of all schemes, K below one stage
    (300, 512, 512, 16),    # 128 x 128 tiled W4A4 and fp8, decode GEMM for the weight-only schemes
    (300, 520, 96, 24),     # decode GEMM for W4A4 (K % 256 != 0), ragged N, rank % 16 != 0
    (257, 300, 544, 128),   # largest rank, ragged everything
    (130, 200, 160, 48),    # decode GEMM W4A4, few-token fp8
    (16, 8200, 512, 24),    # few-token kernels on a full grid (fewer waves per workgroup), ragged N
]


@pytest.mark.parametrize("M,N,K,rank", ROUTE_SHAPES)
@pytest.mark.parametrize("scheme,weight_only", SCHEMES)
def test_lora_matches_oracle(scheme, weight_only, M, N, K, rank):
    x, w, a, b = _inputs(M, N, K, rank, rank)
    run_lora(scheme, weight_only, x, w, a, b, SCALE,
             what="%s%s %dx%dx%d r%d" % (scheme, "-wo" if weight_only else "", M, N, K, rank))


# Large tiles, compared on sampled rows: 4096 x 3072 runs W4A4, fp8 and W4A16 on 256 x 192 tiles
# and W8A16 on 128 x 192; 4096 x 4096 runs W4A4 on 256 x 256, fp8 on 128 x 128 (the square
# fp8 tile takes no adapter), W4A16 on 256 x 128 and W8A16 on 128 x 256
BIG_SHAPES = [(4096, 3072, 3072, 32), (4096, 4096, 512, 64)]


@pytest.mark.parametrize("M,N,K,rank", BIG_SHAPES)
@pytest.mark.parametrize("scheme,weight_only", SCHEMES)
def test_lora_large_tiles_sampled(scheme, weight_only, M, N, K, rank):
    x, w, a, b = _inputs(M, N, K, rank, 1)
    run_lora(scheme, weight_only, x, w, a, b, 1.0, sample=64,
             what="%s%s %dx%dx%d r%d" % (scheme, "-wo" if weight_only else "", M, N, K, rank))


# The fp8r W8A8 GEMM copies the tile's rows of T and B into LDS when the rank is a multiple of 8
# up to 32 (else it reads them from global memory in the epilogue): each of its adapter tiles at
# both ranks of that copy and one past it -- 64 x 64 (300 x 520), 64 x 128 (1100 x 1000),
# 128 x 128 (2100 x 1000), 256 x 192 (4096 x 3072); K = 320 is not a whole number of 128-deep
# stages, 512 is.
FP8_TILE_SHAPES = [(300, 520, 320), (1100, 1000, 512), (2100, 1000, 320), (2100, 1000, 512), (4096, 3072, 320)]


@pytest.mark.parametrize("rank", [8, 24, 32, 40])
@pytest.mark.parametrize("M,N,K", FP8_TILE_SHAPES)
def test_fp8r_adapter_tiles(M, N, K, rank):
    x, w, a, b = _inputs(M, N, K, rank, 8)
    run_lora("fp8r", False, x, w, a, b, SCALE, sample=96, what="fp8r %dx%dx%d r%d" % (M, N, K, rank))


# On the hand-ordered 256 x 192 loop (K % 128 == 0), ranks that are multiples of 8 from 40 get T and
# B copied into the stage buffers the last stages leave free: rank values 0..63 into that of the
# second-to-last stage (in the prologue for a single stage), 64..127 into that of the last one;
# 60 and 100 read them from global memory. K = 128 and 256 are the one- and two-stage cases,
# 4000 x 3000 has ragged last tiles.
LATE_SHAPES = [(4096, 3072, 128, 64), (4096, 3072, 256, 40), (4096, 3072, 640, 48), (4000, 3000, 384, 56),
               (4000, 3000, 384, 64), (4096, 3072, 640, 72), (4096, 3072, 640, 60), (4096, 3072, 128, 128),
               (4096, 3072, 256, 96), (4000, 3000, 384, 120), (4096, 3072, 640, 128), (4096, 3072, 640, 100)]


@pytest.mark.parametrize("M,N,K,rank", LATE_SHAPES)
def test_fp8r_adapter_late_copy(M, N, K, rank):
    x, w, a, b = _inputs(M, N, K, rank, 9)
    run_lora("fp8r", False, x, w, a, b, SCALE, sample=96, what="fp8r %dx%dx%d r%d" % (M, N, K, rank))


@pytest.mark.parametrize("M,N,K,rank", ROUTE_SHAPES + [(4096, 3072, 3072, 32), (4096, 3072, 640, 64),
                                            (4096, 3072, 640, 128), (2048, 3072, 512, 16)])
@pytest.mark.parametrize("scheme,weight_only", SCHEMES)
def test_zero_scale_is_the_plain_linear_bit_for_bit(scheme, weight_only, M, N, K, rank):
    x, w, a, b = _inputs(M, N, K, rank, 2)
    flags = L.BSQ_WEIGHT_ONLY if weight_only else 0
    dx, da, db = dev_bf16(x), dev_bf16(a), dev_bf16(b)
    if scheme == "fp8r":
        wq, sw = quant.quantize_fp8r(w)
        plain = L.bsq_gemm_fp8r(dx, dev(wq), dev(sw), flags=flags)
        with_lora = L.bsq_gemm_fp8r_lora(dx, dev(wq), dev(sw), da, db, 0.0, flags=flags)
    else:
        gw = quant.calibrate_global_scale(w)
        wq, sfw = quant.quantize_nvfp4(w, gw)
        gx = None if weight_only else dev_scalar(quant.calibrate_global_scale(x))
        plain = L.bsq_gemm_nvfp4(dx, dev(wq), dev(sfw), dev_scalar(gw), gx, flags=flags)
        with_lora = L.bsq_gemm_nvfp4_lora(dx, dev(wq), dev(sfw), dev_scalar(gw), gx, da, db, 0.0, flags=flags)
    torch.cuda.synchronize()
    assert np.array_equal(host(with_lora), host(plain))


# The down projection alone takes the K-sliced kernel or, with K <= 3072, the whole-row kernel
# without the encoding: for 256-4096 rows (rank 17-32 from 2048 rows), below 256 rows from rank 65;
# with 3072 < K <= 6144 (twelve chunks a wave) from 2048 rows.
DOWN_SHAPES = [(1, 32, 1), (17, 96, 4), (64, 256, 48), (40, 512, 64), (33, 128, 128), (300, 3072, 32),
               (4096, 3072, 32), (77, 12288, 16), (256, 1024, 64), (2048, 544, 24), (512, 96, 128),
               (300, 2048, 100), (1000, 3072, 16), (2048, 4096, 48), (2200, 6144, 16), (1000, 4096, 32)]


@pytest.mark.parametrize("M,K,rank", DOWN_SHAPES)
def test_down_projection(M, K, rank):
    """T = bf16(s X A^T) within bf16 rounding (2^-9) plus fp32 accumulation of the exact value."""
    x = syn.normal_bf16((M, K), 61, M + K)
    a, _ = syn.lora_adapter(61, rank, 8, K, block=rank)
    t = host(L.bsq_lora_down(dev_bf16(x), dev_bf16(a), SCALE))
    torch.cuda.synchronize()
    ref = lora.lora_down(x, a, SCALE)
    got = codec.bf16_to_f64(t)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5 * rms)


def test_down_projection_strided_input_and_determinism():
    M, K, ldx, rank = 70, 256, 320, 24
    xf = syn.normal_bf16((M, ldx), 62, 1)
    a, _ = syn.lora_adapter(62, rank, 8, K)
    xs = dev_bf16(xf)[:, :K]
    t1 = host(L.bsq_lora_down(xs, dev_bf16(a), 2.0))
    t2 = host(L.bsq_lora_down(xs, dev_bf16(a), 2.0))
    torch.cuda.synchronize()
    assert np.array_equal(t1, t2)
    ref = lora.lora_down(np.ascontiguousarray(xf[:, :K]), a, 2.0)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    assert np.all(np.abs(codec.bf16_to_f64(t1) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5 * rms)


def test_empty_batch_is_a_noop():
    w = torch.zeros((64, 64), dtype=torch.uint8, device="cuda")
    s = torch.ones((64,), dtype=torch.float32, device="cuda")
    a = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((64, 8), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    y = L.bsq_gemm_fp8r_lora(x, w, s, a, b, 1.0)
    assert y.shape == (0, 64)


# The K-sliced kernel (20 x 512 r32, 130 x 160 r48, 5000 x 1024 r32) or the whole-row kernel
# (the others) writes the encoding.
@pytest.mark.parametrize("M,N,K,rank", [(300, 512, 512, 16), (4096, 3072, 3072, 32), (20, 1024, 512, 32),
                                        (130, 200, 160, 48), (257, 300, 544, 128), (16, 256, 96, 100),
                                        (5000, 256, 1024, 16), (5000, 256, 1024, 32), (2048, 256, 4608, 64)])
def test_quantized_activations_in_the_workspace_match_the_quantizer(M, N, K, rank):
    """The W4A4 path encodes X to nvfp4 inside its down projection: the workspace's first two
    parts (packed codes, then block scales, each padded to 256 bytes) must equal the activation
    quantizer's output bit for bit, and the linear must match the oracle."""
    x, w, a, b = _inputs(M, N, K, rank, 3)
    gw = quant.calibrate_global_scale(w)
    wq, sfw = quant.quantize_nvfp4(w, gw)
    gx = dev_scalar(quant.calibrate_global_scale(x))
    dx = dev_bf16(x)
    nbytes = L.bsq_lora_workspace_bytes(L.BSQ_FMT_NVFP4, M, N, K, rank)
    ws = torch.zeros((nbytes,), dtype=torch.uint8, device="cuda")
    y = L.bsq_gemm_nvfp4_lora(dx, dev(wq), dev(sfw), dev_scalar(gw), gx, dev_bf16(a), dev_bf16(b), SCALE,
                              workspace=ws)
    xq, xs = L.bsq_quantize_act_nvfp4(dx, gx)
    torch.cuda.synchronize()
    pad = lambda n: (n + 255) // 256 * 256
    got = host(ws)
    assert np.array_equal(got[:M * K // 2], host(xq).reshape(-1))
    off = pad(M * K // 2)
    assert np.array_equal(got[off:off + M * K // 16], host(xs).reshape(-1))
    rows = _rows_subset(M, 300, 11)
    gxh = quant.calibrate_global_scale(x)
    xq_o, sfx_o = quant.quantize_nvfp4(x[rows], gxh)
    ref = lora.lora_linear(gemm.gemm_nvfp4(xq_o, sfx_o, gxh, wq, sfw, gw), x[rows], a, b, SCALE)
    assert_gemm_close(host(y)[rows], ref, "nvfp4 %dx%dx%d r%d" % (M, N, K, rank),
                      extra=t_rounding_bound(x[rows], a, b, SCALE))


# fp8r linears encode X and compute T in one kernel (16 whole rows a workgroup, up to 8 waves of
# 384 K values) for K <= 3072 up to 4096 rows, and beyond that at rank <= 16; for 3072 < K <= 6144
# (768 K values a wave) from 2048 rows; otherwise the quantizer and the K-sliced projection run. Shapes: one wave with a half chunk (K = 96), ragged
# rows, 2 waves with a partial last chunk (K = 544), a full workgroup (K = 3072) at 4096 tokens,
# 5000 tokens on both paths, the unfused path for long rows below 2048 tokens (40 x 4096), and
# twelve chunks a wave from 2048 tokens (K = 3104, 4096, 6144).
@pytest.mark.parametrize("M,N,K,rank", [(1, 64, 96, 5), (33, 128, 544, 16), (300, 256, 1056, 48),
                                        (4096, 3072, 3072, 32), (70, 256, 3072, 128), (40, 128, 4096, 24),
                                        (5000, 256, 1024, 16), (5000, 256, 1024, 32), (2048, 256, 4096, 32),
                                        (2100, 128, 6144, 128), (2048, 256, 3104, 16)])
def test_fp8r_workspace_holds_the_quantizer_output_and_t(M, N, K, rank):
    """The fp8r W8A8 adapter path leaves in its workspace X's fp8r codes and row scales (bit for
    bit what the activation quantizer writes) and T = bf16(s X A^T) (within the down
    projection's bound), whichever kernels produced them."""
    x, w, a, b = _inputs(M, N, K, rank, 4)
    wq, sw = quant.quantize_fp8r(w)
    dx = dev_bf16(x)
    nbytes = L.bsq_lora_workspace_bytes(L.BSQ_FMT_FP8R, M, N, K, rank)
    ws = torch.zeros((nbytes,), dtype=torch.uint8, device="cuda")
    L.bsq_gemm_fp8r_lora(dx, dev(wq), dev(sw), dev_bf16(a), dev_bf16(b), SCALE, workspace=ws)
    xq, sx = L.bsq_quantize_act_fp8r(dx)
    torch.cuda.synchronize()
    pad = lambda n: (n + 255) // 256 * 256
    got = host(ws)
    assert np.array_equal(got[:M * K], host(xq).reshape(-1))
    off = pad(M * K)
    assert np.array_equal(got[off:off + 4 * M].view(np.float32), host(sx).reshape(-1))
    toff = L.bsq_gemm_workspace_bytes(L.BSQ_FMT_FP8R, M, N, K)
    t = got[toff:toff + 2 * M * rank].view(np.uint16).reshape(M, rank)
    ref = lora.lora_down(x, a, SCALE)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    assert np.all(np.abs(codec.bf16_to_f64(t) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5 * rms)


def test_fp8r_fused_path_strided_input_and_determinism():
    """The whole-row kernel reads X through its leading dimension (a column slice of a wider
    tensor) and gives the same bits twice; the linear matches the oracle."""
    M, N, K, ldx, rank = 45, 192, 1024, 1280, 20
    xf = syn.normal_bf16((M, ldx), 63, 2)
    w = syn.normal_bf16((N, K), 63, 3, sigma=0.02)
    a, b = syn.lora_adapter(63, rank, N, K)
    x = np.ascontiguousarray(xf[:, :K])
    wq, sw = quant.quantize_fp8r(w)
    dx = dev_bf16(xf)[:, :K]
    y1 = host(L.bsq_gemm_fp8r_lora(dx, dev(wq), dev(sw), dev_bf16(a), dev_bf16(b), SCALE))
    y2 = host(L.bsq_gemm_fp8r_lora(dx, dev(wq), dev(sw), dev_bf16(a), dev_bf16(b), SCALE))
    torch.cuda.synchronize()
    assert np.array_equal(y1, y2)
    xq, sx = quant.quantize_fp8r(x)
    ref = lora.lora_linear(gemm.gemm_fp8r(xq, sx, wq, sw), x, a, b, SCALE)
    assert_gemm_close(y1, ref, "fp8r strided x", extra=t_rounding_bound(x, a, b, SCALE))


def test_nvfp4_whole_row_path_strided_input():
    """The nvfp4 linear's whole-row down projection (300 rows, rank 16) reads X through its
    leading dimension, encodes it as the quantizer does and matches the oracle."""
    M, N, K, ldx, rank = 300, 256, 512, 640, 16
    xf = syn.normal_bf16((M, ldx), 64, 4)
    w = syn.normal_bf16((N, K), 64, 5, sigma=0.02)
    a, b = syn.lora_adapter(64, rank, N, K)
    x = np.ascontiguousarray(xf[:, :K])
    gw = quant.calibrate_global_scale(w)
    wq, sfw = quant.quantize_nvfp4(w, gw)
    gxh = quant.calibrate_global_scale(x)
    dx = dev_bf16(xf)[:, :K]
    nbytes = L.bsq_lora_workspace_bytes(L.BSQ_FMT_NVFP4, M, N, K, rank)
    ws = torch.zeros((nbytes,), dtype=torch.uint8, device="cuda")
    y = L.bsq_gemm_nvfp4_lora(dx, dev(wq), dev(sfw), dev_scalar(gw), dev_scalar(gxh), dev_bf16(a), dev_bf16(b),
                              SCALE, workspace=ws)
    torch.cuda.synchronize()
    xq_o, sfx_o = quant.quantize_nvfp4(x, gxh)
    got = host(ws)
    assert np.array_equal(got[:M * K // 2], xq_o.reshape(-1))
    ref = lora.lora_linear(gemm.gemm_nvfp4(xq_o, sfx_o, gxh, wq, sfw, gw), x, a, b, SCALE)
    assert_gemm_close(host(y), ref, "nvfp4 strided x", extra=t_rounding_bound(x, a, b, SCALE))
