"""Pins for the oracle codecs: value sets, nearest-even rounding, bf16, packing.

Each test checks oracle.codec against something other than itself: the
format definitions (hand-written fixtures), a brute-force nearest-grid search,
exact midpoints, monotonicity, or exact rational rounding.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codec
from tests.golden_io import code_value_table, lines, value_code_table


def f32(x):
    return np.float64(np.float32(x))


# ---- value sets ---------------------------------------------------------------

def test_e2m1_value_set_matches_fixture():
    codes, vals = code_value_table("e2m1_values.txt")
    got = codec.e2m1_decode(codes)
    assert np.array_equal(got, vals)
    assert np.array_equal(np.signbit(got), np.signbit(vals))  # 0x8 is -0
    assert set(np.abs(got)) == {0, 0.5, 1, 1.5, 2, 3, 4, 6}


def test_e4m3_anchors_match_fixture():
    codes, vals = code_value_table("e4m3_anchors.txt")
    got = codec.e4m3_decode(codes)
    nan = np.isnan(vals)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], vals[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(vals[~nan]))


def test_e4m3_table_structure():
    t = codec.E4M3_TABLE
    finite = t[~np.isnan(t)]
    assert np.sum(np.isnan(t)) == 2 and np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert finite.max() == 448 and finite.min() == -448
    assert len(set(np.abs(finite))) == 127          # 0 plus 126 distinct magnitudes
    assert np.all(np.diff(t[:0x7F]) > 0)             # codes 0x00..0x7E increase
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])
    # the E2M1 values are all E4M3 values (an nvfp4 decode fits in e4m3 * e4m3)
    assert set(codec.e2m1_decode(np.arange(8))) <= set(finite)


# ---- brute-force nearest-grid rounding ---------------------------------------

def _brute_encode(v, grid_vals, grid_codes, sign_bit, vmax):
    """Nearest grid value by exhaustive search; ties go to the code with even LSB."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    d = np.abs(a[:, None] - grid_vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = (grid_codes[None, :] & 1) == 0
    pick_even = cand & even
    idx = np.where(pick_even.any(axis=1), pick_even.argmax(axis=1), cand.argmax(axis=1))
    code = grid_codes[idx]
    code = np.where(a >= vmax, grid_codes[np.argmax(grid_vals)], code)
    return (code | np.where(np.signbit(v), sign_bit, 0)).astype(np.uint8)


E4M3_GRID_CODES = np.arange(0x7F)
E4M3_GRID_VALS = codec.e4m3_decode(E4M3_GRID_CODES)
E2M1_GRID_CODES = np.arange(8)
E2M1_GRID_VALS = codec.e2m1_decode(E2M1_GRID_CODES)


def _all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        v = (b << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    return v[np.isfinite(v)]


@pytest.mark.parametrize("scale", [1.0, 3.0, 2.0 ** -7, 448.0 / 3.0])
def test_e4m3_rounding_exhaustive_bf16_times_scale(scale):
    v = codec.rn32(_all_finite_bf16() * f32(scale))
    v = v[np.isfinite(v)]
    for chunk in np.array_split(v, 16):
        got = codec.encode_e4m3(chunk)
        ref = _brute_encode(chunk, E4M3_GRID_VALS, E4M3_GRID_CODES, 0x80, 448.0)
        assert np.array_equal(got, ref)


@pytest.mark.parametrize("scale", [1.0, 3.0, 2.0 ** -7, 448.0 / 3.0])
def test_e2m1_rounding_exhaustive_bf16_times_scale(scale):
    v = codec.rn32(_all_finite_bf16() * f32(scale))
    v = v[np.isfinite(v)]
    got = codec.encode_e2m1(v)
    ref = _brute_encode(v, E2M1_GRID_VALS, E2M1_GRID_CODES, 0x8, 6.0)
    assert np.array_equal(got, ref)


def _midpoint_cases(grid):
    g = np.sort(np.unique(np.abs(grid)))
    mids = (g[:-1] + g[1:]) / 2          # exact: grid values are short dyadics
    lo = np.nextafter(mids.astype(np.float32), np.float32(-np.inf)).astype(np.float64)
    hi = np.nextafter(mids.astype(np.float32), np.float32(np.inf)).astype(np.float64)
    return g, mids, lo, hi


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_rounding_at_every_midpoint_and_one_ulp_off(fmt):
    if fmt == "e4m3":
        grid, enc, dec = E4M3_GRID_VALS, codec.encode_e4m3, codec.e4m3_decode
    else:
        grid, enc, dec = E2M1_GRID_VALS, codec.encode_e2m1, codec.e2m1_decode
    g, mids, lo, hi = _midpoint_cases(grid)
    assert np.all(mids == codec.rn32(mids))   # every midpoint is an fp32 value
    for sign in (1.0, -1.0):
        assert np.array_equal(np.abs(dec(enc(sign * lo))), g[:-1])
        assert np.array_equal(np.abs(dec(enc(sign * hi))), g[1:])
        at = enc(sign * mids)
        assert np.all((at & 1) == 0)         # ties land on the even code
        assert np.all((np.abs(dec(at)) == g[:-1]) | (np.abs(dec(at)) == g[1:]))


def test_saturation_and_signed_zero():
    big = np.array([448.0, 449.0, 463.0, 464.0, 465.0, 1e6, 3e38])
    assert np.all(codec.encode_e4m3(big) == 0x7E)
    assert np.all(codec.encode_e4m3(-big) == 0xFE)
    assert np.all(codec.encode_e2m1(np.array([6.0, 6.9, 7.0, 1e9])) == 0x7)
    assert np.all(codec.encode_e2m1(np.array([-6.0, -7.5])) == 0xF)
    tiny = np.array([-0.0, -1e-30, -2.0 ** -11])
    assert np.all(codec.encode_e4m3(tiny) == 0x80)
    assert np.all(codec.encode_e2m1(np.array([-0.0, -0.1, -0.25])) == 0x8)
    assert np.all(codec.encode_e4m3(np.array([0.0, 2.0 ** -11])) == 0x00)


def test_monotone_encode():
    rng = np.random.default_rng(7)
    v = np.sort(codec.rn32(rng.standard_normal(200000) * 100))
    assert np.all(np.diff(codec.e4m3_decode(codec.encode_e4m3(v))) >= 0)
    v2 = np.sort(codec.rn32(rng.standard_normal(200000) * 3))
    assert np.all(np.diff(codec.e2m1_decode(codec.encode_e2m1(v2))) >= 0)


def test_fp8r_row_fixture_codes():
    vals, codes = value_code_table("fp8r_row_worked.txt")
    # the fixture values all lie on the bf16 grid; d = 1 so the codes are plain E4M3 roundings
    assert np.array_equal(codec.encode_e4m3(vals), codes)


# ---- bf16 ---------------------------------------------------------------------

def _bf16_nearest_exact(x32):
    """Nearest bf16 to an fp32 value by exact rational comparison of the two neighbours."""
    (u,) = struct.unpack("<I", struct.pack("<f", x32))
    lo = u & 0xFFFF0000
    hi = lo + 0x10000
    def val(bits):
        return Fraction(struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0])
    x = Fraction(x32)
    dl, dh = abs(x - val(lo)), abs(val(hi) - x) if (hi >> 23) & 0xFF != 0xFF else None
    if dh is None or dl < dh or (dl == dh and ((lo >> 16) & 1) == 0):
        return lo >> 16
    return (hi >> 16) & 0xFFFF


def test_bf16_rne_against_exact_neighbour_search():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000),
                        [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 2.0 ** -130, 65504.0]])
    x = x.astype(np.float32)
    got = codec.f32_to_bf16(x.astype(np.float64))
    ref = np.array([_bf16_nearest_exact(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)
    # torch's own float -> bfloat16 conversion is round-to-nearest-even too
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, tb)


def test_bf16_roundtrip_exact():
    b = np.arange(65536, dtype=np.uint16)
    v = codec.bf16_to_f64(b)
    fin = np.isfinite(v)
    assert np.array_equal(codec.f32_to_bf16(v[fin]), b[fin])


# ---- packing ------------------------------------------------------------------

def test_packing_fixture():
    for ln in lines("packing.txt"):
        lhs, rhs = ln.split(":")
        vals = np.array([float(t) for t in lhs.split()])
        want = np.array([int(t, 16) for t in rhs.split()], dtype=np.uint8)
        got = codec.pack_e2m1(codec.encode_e2m1(vals))
        assert np.array_equal(got, want)


def test_pack_unpack_roundtrip():
    rng = np.random.default_rng(11)
    c = rng.integers(0, 16, size=(7, 64)).astype(np.uint8)
    assert np.array_equal(codec.unpack_e2m1(codec.pack_e2m1(c)), c)
    p = rng.integers(0, 256, size=(5, 32)).astype(np.uint8)
    assert np.array_equal(codec.pack_e2m1(codec.unpack_e2m1(p)), p)
