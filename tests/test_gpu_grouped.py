"""GPU parity of the grouped launch (bsq_gemm_grouped_q).

On the tiled kernels every problem of a group must come out bit for bit as
the single pre-quantized entry point (bsq_gemm_fp8r_q / bsq_gemm_nvfp4_q)
computes it -- the grouped kernels run the same tile code, only the workgroup
-> (problem, tile) mapping differs. On the few-token kernels bit equality is
asserted only for problems whose single call runs the group's workgroup shape
(waves splitting K, activation blocks per workgroup); the others sum the same
products in another order and are held to the oracle's tolerance. Every
grouped call must repeat its own bits, and sampled rows of every problem must
match the oracle's fp64 product within the GEMM tolerance. Groups cover the
grouped tiled kernels (ragged M and N, mixed K, longest K not first), every
few-token variant, mixed routes, the per-problem fallback (too few tiles, a K
the grouped kernels do not take, empty problems) and the four joint-block
linears at 1, 16, 48 and 16384 tokens ("FLUX 3 Image Klein" release page,
section one: 28 joint blocks of qkv, proj, MLP up and down).
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_row_amd import synthetic as syn
from oracle import gemm, quant
from tests.gpu_util import assert_gemm_close, dev_bf16, host

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from block_scaled_precision_row_amd import _lib as L


def _acts(fmt, M, K, block):
    """Seeded activations, quantized on the GPU (bit-exact with the oracle's quantizers)."""
    xb = syn.activations(syn.JOINT_4MP, M, K, block=block)
    x = dev_bf16(xb)
    if fmt == "fp8r":
        return xb, L.bsq_quantize_act_fp8r(x)
    gx = L.bsq_calibrate_global_scale(x)
    xq, xs = L.bsq_quantize_act_nvfp4(x, gx)
    return xb, (xq, xs, gx)


def _weights(fmt, N, K, block):
    wb = syn.weights(syn.JOINT_4MP, N, K, block=block)
    w = dev_bf16(wb)
    if fmt == "fp8r":
        return L.bsq_quantize_act_fp8r(w)
    gw = L.bsq_calibrate_global_scale(w)
    wq, ws = L.bsq_quantize_act_nvfp4(w, gw)
    return wq, ws, gw


def _problem(fmt, xs, ws):
    if fmt == "fp8r":
        return (xs[0], xs[1], ws[0], ws[1])
    return (xs[0], xs[1], xs[2], ws[0], ws[1], ws[2])


def _single(fmt, p):
    return L.bsq_gemm_fp8r_q(*p) if fmt == "fp8r" else L.bsq_gemm_nvfp4_q(*p)


def _fmt(fmt):
    return L.BSQ_FMT_FP8R if fmt == "fp8r" else L.BSQ_FMT_NVFP4


def _oracle_rows(fmt, p, xb, rows):
    """The oracle's product on `rows`, from the weights' codes and scales as the GPU holds them;
    the GPU's encoding of these activation rows must equal the oracle quantizer's."""
    r = torch.as_tensor(rows, device="cuda")
    if fmt == "fp8r":
        xq, sx = host(p[0][r]), host(p[1][r])
        wq, sw = host(p[2]), host(p[3])
        oq, osx = quant.quantize_fp8r(xb[rows])
        assert np.array_equal(oq, xq) and np.array_equal(osx, sx)
        return gemm.gemm_fp8r(xq, sx, wq, sw)
    xq, xs, gx = host(p[0][r]), host(p[1][r]), host(p[2])
    wq, ws, gw = host(p[3]), host(p[4]), host(p[5])
    oq, os_ = quant.quantize_nvfp4(xb[rows], np.float32(gx[0]))
    assert np.array_equal(oq, xq) and np.array_equal(os_, xs)
    return gemm.gemm_nvfp4(xq, xs, np.float32(gx[0]), wq, ws, np.float32(gw[0]))


def _check_group(fmt, probs, xbs, sample=12, seed=0, exact=None):
    """`exact`: the problems whose output must equal the single call's bit for bit (all by default);
    every sampled row of every problem is checked against the oracle."""
    ys = L.bsq_gemm_grouped_q(_fmt(fmt), probs)
    again = L.bsq_gemm_grouped_q(_fmt(fmt), probs)
    singles = [_single(fmt, p) for p in probs]
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    for i, (y, s) in enumerate(zip(ys, singles)):
        yb, sb = host(y), host(s)
        assert np.array_equal(yb, host(again[i])), "problem %d: two grouped calls differ" % i
        if exact is None or i in exact:
            assert np.array_equal(yb, sb), "problem %d differs from its single launch" % i
        if sample:
            M = yb.shape[0]
            rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, sample, replace=False)]))
            assert_gemm_close(yb[rows], _oracle_rows(fmt, probs[i], xbs[i], rows), "%s grouped problem %d" % (fmt, i))
    return ys


@pytest.mark.parametrize("fmt", ["fp8r", "nvfp4"])
def test_grouped_kernel_mixed_shapes(fmt):
    """A grouped tiled grid (592 tiles of 256 x 192: 128 x 128 tiles two to a compute unit), ragged
    M and N, the longest K last."""
    M = 4000
    xb1, x1 = _acts(fmt, M, 1024, 0)
    xb2, x2 = _acts(fmt, M, 2048, 1)
    shapes = [(2304, 1024), (776, 1024), (3072, 1024), (760, 2048)]
    probs, xbs = [], []
    for b, (N, K) in enumerate(shapes):
        probs.append(_problem(fmt, x1 if K == 1024 else x2, _weights(fmt, N, K, 10 + b)))
        xbs.append(xb1 if K == 1024 else xb2)
    _check_group(fmt, probs, xbs)


@pytest.mark.parametrize("fmt", ["fp8r", "nvfp4"])
def test_grouped_fallback_paths(fmt):
    """Groups the grouped kernels do not take run one launch per problem, with the same bits:
    too few tiles (300 and 2000 tokens: less than two rounds of 256 x 192 tiles), a K that is not
    a whole number of the grouped kernels' stages, empty problems."""
    xb, x = _acts(fmt, 300, 512, 2)
    small = [_problem(fmt, x, _weights(fmt, N, 512, 20 + i)) for i, N in enumerate((520, 264))]
    _check_group(fmt, small, [xb, xb])
    xb2, x2 = _acts(fmt, 2000, 1088, 3)  # K % 128 == 64: neither grouped kernel's stage
    odd = [_problem(fmt, x2, _weights(fmt, N, 1088, 30 + i)) for i, N in enumerate((3072, 3000))]
    _check_group(fmt, odd, [xb2, xb2], sample=6)
    # an empty problem (M = 0) among full ones is skipped
    xb3, x3 = _acts(fmt, 2000, 1024, 5)
    e = tuple(t[:0] if t.dim() == 2 or t.numel() > 1 else t for t in x3)  # no rows (global scale kept)
    mixed = [_problem(fmt, x3, _weights(fmt, 3072, 1024, 40)), _problem(fmt, e, _weights(fmt, 256, 1024, 41)),
             _problem(fmt, x3, _weights(fmt, 3072, 1024, 42))]
    ys = L.bsq_gemm_grouped_q(_fmt(fmt), mixed)
    singles = [_single(fmt, mixed[0]), _single(fmt, mixed[2])]
    torch.cuda.synchronize()
    assert ys[1].shape == (0, 256)
    assert np.array_equal(host(ys[0]), host(singles[0])) and np.array_equal(host(ys[2]), host(singles[1]))


@pytest.mark.parametrize("fmt", ["fp8r", "nvfp4"])
@pytest.mark.parametrize("M", [syn.JOINT_TOKENS, 2048, 600, 200])
def test_grouped_joint_block(fmt, M):
    """The joint block's four linears in one launch, as the benchmark times them: at 16384 tokens
    on 256 x 256 tiles, at 2048 on 256 x 192 tiles, at 600 (ragged) on 128 x 128 tiles two to a
    compute unit, at 200 on those tiles for nvfp4 (432 of them) and one launch per problem for
    fp8r."""
    block = 0 if fmt == "nvfp4" else 1
    xb_a, xa = _acts(fmt, M, 3072, 0)
    xb_b, xb = _acts(fmt, M, 12288, 1)
    probs, xbs = [], []
    for gi, (name, N, K) in enumerate(syn.JOINT_GEMMS):
        probs.append(_problem(fmt, xa if K == 3072 else xb, _weights(fmt, N, K, block * 4 + gi)))
        xbs.append(xb_a if K == 3072 else xb_b)
    _check_group(fmt, probs, xbs, sample=4)


@pytest.mark.parametrize("fmt", ["fp8r", "nvfp4"])
@pytest.mark.parametrize("M", [1, 16, 48])
def test_grouped_few_tokens_joint_block(fmt, M):
    """The joint block's four linears for a few tokens as one grid of the few-token kernels (a
    workgroup per 32 weight rows). The group's workgroups split K over eight waves (nvfp4) or
    four (fp8r; eight at one token, and two activation blocks a workgroup at 48 tokens); alone,
    qkv and up (grids of 256 or more weight blocks) take four waves at 16 tokens (nvfp4) and at
    one token (fp8r), and the tiled kernels at 48 tokens, and fp8r's proj and down one block a
    workgroup at 48 tokens. Bit equality is asserted where the shapes agree."""
    xb_a, xa = _acts(fmt, M, 3072, 6)
    xb_b, xb = _acts(fmt, M, 12288, 7)
    probs, xbs = [], []
    for gi, (name, N, K) in enumerate(syn.JOINT_GEMMS):
        probs.append(_problem(fmt, xa if K == 3072 else xb, _weights(fmt, N, K, 50 + gi)))
        xbs.append(xb_a if K == 3072 else xb_b)
    exact = {("nvfp4", 1): None, ("nvfp4", 16): (1, 3), ("nvfp4", 48): (1, 3),
             ("fp8r", 1): (1, 3), ("fp8r", 16): None, ("fp8r", 48): ()}[(fmt, M)]
    _check_group(fmt, probs, xbs, sample=min(M, 6), exact=exact)


@pytest.mark.parametrize("fmt", ["fp8r", "nvfp4"])
# `exact`, per scheme: the problems whose single call runs the group's workgroup shape (waves and
# activation blocks per workgroup), so that their bits must match; None = all of them
@pytest.mark.parametrize("M,shapes,exact", [
    # two activation blocks a workgroup; alone, fp8r's smaller grids take one block a workgroup
    (100, [(4096, 1024), (2048, 1024), (3072, 2048), (2000, 1024)], {"nvfp4": None, "fp8r": (0,)}),
    # a handful of tokens on a small grid (eight waves a workgroup for both schemes)
    (4, [(1024, 1024), (512, 1024), (2048, 1024)], {"nvfp4": None, "fp8r": None}),
    # alone, N = 12288 would take the tiled kernels, and fp8r's N = 3072 one block a workgroup
    (40, [(3072, 3072), (12288, 3072)], {"nvfp4": (0,), "fp8r": ()}),
    # the same past 64 tokens: one launch per problem
    (80, [(3072, 3072), (12288, 3072)], {"nvfp4": None, "fp8r": None}),
])
def test_grouped_few_token_variants(fmt, M, shapes, exact):
    """Few-token groups on each workgroup variant the grouped launch picks, ragged N included, and
    groups whose problems alone take different routes: up to 64 tokens all of them run on the
    few-token kernels (bit for bit the single call where it runs the same workgroup shape, within
    the tolerance of the oracle everywhere), beyond that one launch per problem."""
    exact = exact[fmt]
    xbs, probs, acts = [], [], {}
    for b, (N, K) in enumerate(shapes):
        if K not in acts:
            acts[K] = _acts(fmt, M, K, 60 + len(acts))
        xb, x = acts[K]
        probs.append(_problem(fmt, x, _weights(fmt, N, K, 70 + b)))
        xbs.append(xb)
    _check_group(fmt, probs, xbs, sample=min(M, 6), exact=exact)


@pytest.mark.parametrize("fmt", ["fp8r", "nvfp4"])
@pytest.mark.parametrize("M", [1, 16, 40])
def test_grouped_weight_only_joint_block(fmt, M):
    """Weight-only linears (bf16 activations, the fallback's arithmetic) grouped: the joint block's
    four linears. At 1 and 16 tokens every problem is on the few-token route and the group runs as
    one grid of eight-wave (nvfp4) or four-wave (fp8r) workgroups, the shape proj and down take
    alone (qkv and up, with grids of 256 or more weight blocks, take four or two waves alone); at
    40 tokens qkv and up alone take the tiled kernels, so the group runs one launch per problem."""
    xs = {K: syn.activations(syn.JOINT_4MP, M, K, block=8 + (K > 3072)) for K in (3072, 12288)}
    xd = {K: dev_bf16(v) for K, v in xs.items()}
    probs, host_w = [], []
    for gi, (name, N, K) in enumerate(syn.JOINT_GEMMS):
        w = _weights(fmt, N, K, 80 + gi)
        probs.append((xd[K],) + tuple(w))
        host_w.append(tuple(host(t) for t in w))
    ys = L.bsq_gemm_grouped_weight_only(_fmt(fmt), probs)
    again = L.bsq_gemm_grouped_weight_only(_fmt(fmt), probs)
    if fmt == "fp8r":
        singles = [L.bsq_gemm_fp8r(p[0], p[1], p[2], flags=L.BSQ_WEIGHT_ONLY) for p in probs]
    else:
        singles = [L.bsq_gemm_nvfp4(p[0], p[1], p[2], p[3], None, flags=L.BSQ_WEIGHT_ONLY) for p in probs]
    torch.cuda.synchronize()
    exact = None if M == 40 else (1, 3)
    rng = np.random.default_rng(M)
    for i, (name, N, K) in enumerate(syn.JOINT_GEMMS):
        yb = host(ys[i])
        assert np.array_equal(yb, host(again[i])), "problem %d: two grouped calls differ" % i
        if exact is None or i in exact:
            assert np.array_equal(yb, host(singles[i])), "problem %d differs from its single launch" % i
        rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 6), replace=False)]))
        if fmt == "fp8r":
            ref = gemm.gemm_fp8r_weight_only(xs[K][rows], host_w[i][0], host_w[i][1])
        else:
            ref = gemm.gemm_nvfp4_weight_only(xs[K][rows], host_w[i][0], host_w[i][1], np.float32(host_w[i][2][0]))
        assert_gemm_close(yb[rows], ref, "%s weight-only grouped problem %d" % (fmt, i))
