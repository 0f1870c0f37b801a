"""Pins for the oracle quantizers, calibration and dequantization.

Checked against hand-worked fixtures, the power-of-two special case (where
every scale is exact and quantization reduces to plain nearest-even rounding
onto the grid, found here by brute-force search), invariants that follow from
the definitions (the row / block maximum lands on the format maximum, scale
equivariance, column-permutation equivariance) and error bounds.
"""
import numpy as np
import pytest

from oracle import codec, dequant, quant
from tests.golden_io import directives, lines, value_code_table


def bf16(vals):
    return codec.f32_to_bf16(np.asarray(vals, np.float64))


def brute_nearest(v, grid_vals, grid_codes, sign_bit):
    a = np.abs(v)[:, None]
    d = np.abs(a - grid_vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = cand & ((grid_codes[None, :] & 1) == 0)
    idx = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return grid_codes[idx] | np.where(np.signbit(v), sign_bit, 0)


E2M1_CODES = np.arange(8)
E2M1_VALS = codec.e2m1_decode(E2M1_CODES)
E4M3_CODES = np.arange(0x7F)
E4M3_VALS = codec.e4m3_decode(E4M3_CODES)


def rand_bf16(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return bf16(rng.standard_normal(shape) * scale)


# ---- fp8r ---------------------------------------------------------------------

def test_fp8r_worked_row():
    vals, codes = value_code_table("fp8r_row_worked.txt")
    q, d = quant.quantize_fp8r(bf16(vals)[None, :])
    assert float(d[0]) == float(directives("fp8r_row_worked.txt")["row_scale"])
    assert np.array_equal(q[0], codes)


def test_fp8r_worked_row_with_inexact_reciprocal():
    # d is not a power of two, so fp32(1 / d) is inexact and multiplying by it lands on
    # the other side of E4M3 midpoints than dividing by d would
    name = "fp8r_row_reciprocal_worked.txt"
    vals, codes = value_code_table(name)
    q, d = quant.quantize_fp8r(bf16(vals)[None, :])
    assert float(d[0]) == float(directives(name)["row_scale"])
    assert np.array_equal(q[0], codes)


def test_fp8r_power_of_two_rows_reduce_to_plain_rounding():
    rng = np.random.default_rng(5)
    for k in (-20, -3, 0, 4, 11):
        x = codec.bf16_to_f64(bf16(rng.standard_normal(256) * 2.0 ** k * 100))
        x = np.clip(x, -448 * 2.0 ** k, 448 * 2.0 ** k)
        x[17] = -448.0 * 2.0 ** k                   # row max = 448 * 2^k exactly
        q, d = quant.quantize_fp8r(bf16(x)[None, :])
        assert float(d[0]) == 2.0 ** k
        ref = brute_nearest(x * 2.0 ** -k, E4M3_VALS, E4M3_CODES, 0x80)
        assert np.array_equal(q[0], ref)


def test_fp8r_row_max_lands_on_448_and_error_bound():
    x = rand_bf16((64, 512), 1, 3.0)
    q, d = quant.quantize_fp8r(x)
    xv = codec.bf16_to_f64(x)
    imax = np.argmax(np.abs(xv), axis=1)
    assert np.all(q[np.arange(64), imax] & 0x7F == 0x7E)   # the row maximum encodes to +-448
    assert np.array_equal(d, codec.rn32(np.abs(xv).max(axis=1) / 448).astype(np.float32))
    xh = dequant.fp8r_values(q, d)
    dd = d.astype(np.float64)[:, None]
    bound = (2.0 ** -4 * np.abs(xv) + 2.0 ** -10 * dd) * (1 + 2.0 ** -20)
    assert np.all(np.abs(xv - xh) <= bound)
    assert np.array_equal(np.signbit(xh) & (xh != 0), np.signbit(xv) & (xh != 0))


def test_fp8r_equivariance_and_zero_rows():
    x = rand_bf16((8, 96), 2)
    q, d = quant.quantize_fp8r(x)
    # power-of-two scaling of the input scales d and leaves the codes
    q2, d2 = quant.quantize_fp8r(bf16(codec.bf16_to_f64(x) * 2.0 ** 7))
    assert np.array_equal(q2, q) and np.array_equal(d2, d * np.float32(2.0 ** 7))
    # negation flips sign bits only
    qn, dn = quant.quantize_fp8r(bf16(-codec.bf16_to_f64(x)))
    assert np.array_equal(qn, q ^ 0x80) and np.array_equal(dn, d)
    # permuting columns permutes codes; rows are independent
    perm = np.random.default_rng(0).permutation(96)
    qp, dp = quant.quantize_fp8r(x[:, perm])
    assert np.array_equal(qp, q[:, perm]) and np.array_equal(dp, d)
    qr, dr = quant.quantize_fp8r(x[::-1])
    assert np.array_equal(qr, q[::-1]) and np.array_equal(dr, d[::-1])
    z = bf16(np.array([[0.0, -0.0, 0.0, -0.0]]))
    qz, dz = quant.quantize_fp8r(z)
    assert dz[0] == 0 and list(qz[0]) == [0x00, 0x80, 0x00, 0x80]


# ---- nvfp4 --------------------------------------------------------------------

def test_nvfp4_worked_block():
    vals, codes = value_code_table("nvfp4_block_worked.txt")
    packed, sf = quant.quantize_nvfp4(bf16(vals)[None, :], np.float32(1.0))
    assert sf[0, 0] == int(directives("nvfp4_block_worked.txt")["scale_code"], 16)
    assert np.array_equal(codec.unpack_e2m1(packed)[0], codes)


def test_nvfp4_worked_blocks_with_inexact_global_reciprocal():
    # g is not a power of two: the order of the scale and encode-multiplier steps decides a
    # scale code (line 1) and an element code (line 2)
    for ln in lines("nvfp4_global_reciprocal_worked.txt"):
        parts = ln.split()
        g, sf_code = np.float32(float.fromhex(parts[0])), int(parts[1], 16)
        pairs = [(float(a), int(b, 16)) for a, b in (p.split(":") for p in parts[2:])]
        block = np.zeros(16)
        block[: len(pairs)] = [v for v, _ in pairs]
        assert np.max(np.abs(block)) == pairs[0][0]
        packed, sf = quant.quantize_nvfp4(bf16(block)[None, :], g)
        assert sf[0, 0] == sf_code, (parts[0], hex(sf[0, 0]))
        got = codec.unpack_e2m1(packed)[0]
        assert [int(c) for c in got[: len(pairs)]] == [c for _, c in pairs], parts[0]


def test_nvfp4_saturation_worked():
    for ln in lines("nvfp4_saturation_worked.txt"):
        parts = ln.split()
        amax, sf_code = float(parts[0]), int(parts[1], 16)
        pairs = [(float(a), int(b, 16)) for a, b in (p.split(":") for p in parts[2:])]
        block = np.zeros(16)
        for i, (v, _) in enumerate(pairs):
            block[i] = v
        block[15] = 0.0
        assert np.max(np.abs(block)) == amax
        packed, sf = quant.quantize_nvfp4(bf16(block)[None, :], np.float32(1.0))
        assert sf[0, 0] == sf_code
        got = codec.unpack_e2m1(packed)[0]
        for i, (_, c) in enumerate(pairs):
            assert got[i] == c, (amax, i)


@pytest.mark.parametrize("j", [-10, -3, 0, 2])
def test_nvfp4_power_of_two_scales_reduce_to_plain_rounding(j):
    """g = 2^j and block maxima 6 * 2^m * g: every scale is exact, codes are nearest-even of x 2^-(m+j)."""
    rng = np.random.default_rng(100 + j)
    R, nb = 4, 8
    g = np.float32(2.0 ** j)
    x = np.empty((R, nb * 16))
    ms = rng.integers(-6, 8, size=(R, nb))
    for r in range(R):
        for b in range(nb):
            lim = 6.0 * 2.0 ** (ms[r, b] + j)
            blk = codec.bf16_to_f64(bf16(rng.uniform(-lim, lim, 16)))
            blk[rng.integers(16)] = lim * (1 if rng.random() < 0.5 else -1)
            x[r, b * 16:(b + 1) * 16] = blk
    packed, sf = quant.quantize_nvfp4(bf16(x), g)
    assert np.array_equal(codec.e4m3_decode(sf), 2.0 ** ms.astype(np.float64))
    scale = np.repeat(2.0 ** (ms + j).astype(np.float64), 16, axis=1)
    ref = brute_nearest((x / scale).ravel(), E2M1_VALS, E2M1_CODES, 0x8).reshape(x.shape)
    assert np.array_equal(codec.unpack_e2m1(packed), ref)


def test_nvfp4_block_max_lands_on_6_and_error_bound():
    x = rand_bf16((32, 256), 9, 2.0)
    g = quant.calibrate_global_scale(x)
    packed, sf = quant.quantize_nvfp4(x, g)
    codes = codec.unpack_e2m1(packed)
    xv = codec.bf16_to_f64(x)
    blocks = np.abs(xv).reshape(32, 16, 16)
    imax = blocks.argmax(axis=-1)
    cb = codes.reshape(32, 16, 16)
    normal = codec.e4m3_decode(sf) >= 2.0 ** -6
    top = np.take_along_axis(cb, imax[..., None], axis=-1)[..., 0] & 7
    assert np.all(top[normal] == 7)          # each block's maximum encodes to +-6
    # the tensor maximum's block gets the largest block scale 448
    r, b = np.unravel_index(np.argmax(blocks.max(axis=-1)), (32, 16))
    assert sf[r, b] == 0x7E
    # dequantization error: half an E2M1 spacing (at most 1 in units of sf*g) per element
    xh = dequant.nvfp4_values(packed, sf, g)
    sg = np.repeat(codec.e4m3_decode(sf), 16, axis=1) * np.float64(g)
    assert np.all(np.abs(xv - xh) <= 1.0 * sg * (1 + 2.0 ** -18) + 0.07 * np.abs(xv))


def test_nvfp4_equivariance_and_zero_blocks():
    x = rand_bf16((4, 64), 4)
    g = np.float32(0.0123)
    p, s = quant.quantize_nvfp4(x, g)
    # doubling both the input and the global scale changes nothing
    p2, s2 = quant.quantize_nvfp4(bf16(codec.bf16_to_f64(x) * 2), np.float32(2 * 0.0123))
    assert np.array_equal(p, p2) and np.array_equal(s, s2)
    # negation flips every sign bit
    pn, sn = quant.quantize_nvfp4(bf16(-codec.bf16_to_f64(x)), g)
    assert np.array_equal(codec.unpack_e2m1(pn), codec.unpack_e2m1(p) ^ 8) and np.array_equal(sn, s)
    # permuting whole blocks permutes scales and codes
    perm = np.array([2, 0, 3, 1])
    cols = (perm[:, None] * 16 + np.arange(16)).ravel()
    pp, sp = quant.quantize_nvfp4(x[:, cols], g)
    assert np.array_equal(sp, s[:, perm])
    assert np.array_equal(codec.unpack_e2m1(pp), codec.unpack_e2m1(p)[:, cols])
    z = np.zeros((1, 32))
    z[0, 1::2] = -0.0
    z[0, 20] = 1.5
    pz, sz = quant.quantize_nvfp4(bf16(z), np.float32(0.5))
    cz = codec.unpack_e2m1(pz)[0]
    assert sz[0, 0] == 0 and list(cz[:16]) == [0, 8] * 8
    assert sz[0, 1] != 0


def test_nvfp4_runtime_saturation_beyond_calibration():
    x = rand_bf16((2, 32), 8)
    g = np.float32(1e-4)   # far too small for this data: scales and codes saturate
    p, s = quant.quantize_nvfp4(x, g)
    assert np.all(s == 0x7E)
    xv = codec.bf16_to_f64(x)
    c = codec.unpack_e2m1(p)
    top = 6.0 * 448.0 * np.float64(g)          # largest representable magnitude
    beyond = np.abs(xv) >= top * (1 + 2.0 ** -20)
    assert beyond.sum() > 10 and np.all(c[beyond] & 7 == 7)
    assert np.all(np.abs(dequant.nvfp4_values(p, s, g)) <= top * (1 + 2.0 ** -20))


def test_calibration_definition():
    x = bf16(np.array([[0.5, -2688.0, 3.0], [1.0, 2.0, -4.0]]))
    assert quant.calibrate_global_scale(x) == np.float32(1.0)
    assert quant.calibrate_global_scale(bf16(np.zeros((3, 4)))) == np.float32(1.0)
    y = bf16(np.array([[1.0, -3.0]]))
    assert quant.calibrate_global_scale(y) == np.float32(3.0 / 2688.0)


# ---- dequant to bf16 ----------------------------------------------------------

def test_dequant_bf16_is_rounded_exact_value():
    x = rand_bf16((16, 128), 12, 0.02)
    g = quant.calibrate_global_scale(x)
    p, s = quant.quantize_nvfp4(x, g)
    exact = dequant.nvfp4_values(p, s, g)
    w = codec.bf16_to_f64(dequant.dequant_nvfp4_bf16(p, s, g))
    # bf16 has 8 significant bits: unit roundoff 2^-8, plus the fp32 step
    assert np.all(np.abs(w - exact) <= (2.0 ** -8 + 2.0 ** -23) * np.abs(exact))
    q, d = quant.quantize_fp8r(x)
    w8 = codec.bf16_to_f64(dequant.dequant_fp8r_bf16(q, d))
    e8 = dequant.fp8r_values(q, d)
    assert np.all(np.abs(w8 - e8) <= (2.0 ** -8 + 2.0 ** -23) * np.abs(e8))
    # with power-of-two scales the products are bf16-exact already
    p2, s2 = quant.quantize_nvfp4(x, np.float32(2.0 ** -12))
    assert np.array_equal(codec.bf16_to_f64(dequant.dequant_nvfp4_bf16(p2, s2, np.float32(2.0 ** -12))),
                          dequant.nvfp4_values(p2, s2, np.float32(2.0 ** -12)))


def test_storage_bytes_per_parameter():
    """nvfp4 stores N*K/2 code bytes + N*K/16 scale bytes; fp8r N*K + 4N.

    Cross-check against the pages' file sizes: a 5.6B-parameter generator is
    11.10-11.2 GB in bf16 and 5.6 GB in FP8 ("FLUX 3 Image Klein vs
    Qwen-Image-2.1" memory section and the Klein precision table), i.e. 2 and
    1 bytes per parameter.
    """
    N, K = 3072, 3072
    x = rand_bf16((N // 64, K), 1, 0.02)
    p, s = quant.quantize_nvfp4(x, quant.calibrate_global_scale(x))
    q, d = quant.quantize_fp8r(x)
    n = x.size
    assert p.nbytes + s.nbytes == n // 2 + n // 16
    assert (p.nbytes + s.nbytes) / n == 0.5625
    assert q.nbytes + d.nbytes == n + 4 * x.shape[0]
    params = 5.6e9
    assert abs(params * 2 / 1e9 - 11.2) < 0.15 and abs(params * 1 / 1e9 - 5.6) < 0.01
