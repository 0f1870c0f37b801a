"""Oracle codecs: E2M1 and E4M3 (OCP "FN") value sets, encoders, bf16, nibble packing.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Formats ("BFL (fp8r / nvfp4)", scheme list): fp8r codes are E4M3; nvfp4 codes
are E2M1 packed two per byte with E4M3 block scales.

* E2M1: sign | 2-bit exponent (bias 1) | 1-bit mantissa. Magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}; code 8 is -0. No Inf, no NaN.
* E4M3 (FN variant): sign | 4-bit exponent (bias 7) | 3-bit mantissa.
  Normals (1 + m/8) 2^(e-7), subnormals m 2^-9, max 448 (0x7E),
  0x7F / 0xFF are NaN, no Inf.

Encoding reading (the pages give only the formats): round to nearest, ties to
the even code, saturate finite overflow to the largest magnitude, keep the
sign of zero. Encoders take float64 arrays whose values are exactly
representable in fp32 (results of an fp32 operation) and compute the nearest
grid point as rint(v / q) * q with q the spacing of v's binade -- inside a
binade the integer n = v / q has the parity of the mantissa LSB, so numpy's
round-half-even equals ties-to-even-code.
"""

import numpy as np

E2M1_MAX = 6.0
E4M3_MAX = 448.0

# magnitudes of E2M1 codes 0..7, straight from the field definition
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_decode(codes):
    """Value of each 4-bit E2M1 code (bit 3 = sign)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    mag = _E2M1_MAG[c & 7]
    return np.where(c & 8, -mag, mag)


def _e4m3_field_value(code):
    s, e, m = (code >> 7) & 1, (code >> 3) & 0xF, code & 7
    if e == 15 and m == 7:
        return np.nan
    v = (1.0 + m / 8.0) * 2.0 ** (e - 7) if e else (m / 8.0) * 2.0 ** -6
    return -v if s else v


E4M3_TABLE = np.array([_e4m3_field_value(c) for c in range(256)], dtype=np.float64)
# codes 0x00..0x7E in increasing value order
_E4M3_POS = E4M3_TABLE[:0x7F].copy()


def e4m3_decode(codes):
    """Value of each 8-bit E4M3 code (NaN for 0x7F / 0xFF)."""
    return E4M3_TABLE[np.asarray(codes).astype(np.int64) & 0xFF]


def rn32(x):
    """Round float64 values to the nearest fp32 value (ties to even), returned as float64.

    One fp32 operation on fp32 operands is emulated by computing it in fp64 and
    calling this: double rounding is innocuous for +, -, *, / at these
    precisions (53 >= 2*24 + 2).
    """
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def encode_e4m3(v):
    """fp32 values -> E4M3 codes (uint8), nearest-even, saturating, sign-preserving."""
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)  # values above 448 all end at 448
    _, ex = np.frexp(a)  # a = f * 2^ex, f in [0.5, 1)
    e = ex.astype(np.int64) - 1  # floor(log2 a) for a > 0
    q = np.where(a >= 2.0 ** -6, np.ldexp(1.0, (np.maximum(e, -6) - 3).astype(np.int32)), 2.0 ** -9)
    mag = np.minimum(np.rint(a / q) * q, E4M3_MAX)
    code = np.searchsorted(_E4M3_POS, mag).astype(np.int64)
    assert np.all(_E4M3_POS[code] == mag), "E4M3 grid lookup failed"
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def encode_e2m1(v):
    """fp32 values -> E2M1 codes (uint8 in 0..15), nearest-even, saturating, sign-preserving."""
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E2M1_MAX)
    q = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    mag = np.minimum(np.rint(a / q) * q, E2M1_MAX)
    code = np.searchsorted(_E2M1_MAG, mag).astype(np.int64)
    assert np.all(_E2M1_MAG[code] == mag), "E2M1 grid lookup failed"
    return (code | np.where(neg, 8, 0)).astype(np.uint8)


def bf16_to_f64(bits):
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f32_to_bf16(x):
    """fp32 values -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def pack_e2m1(codes):
    """[..., K] 4-bit codes -> [..., K/2] bytes; element 2j in the low nibble, 2j+1 in the high."""
    c = np.asarray(codes).astype(np.uint8) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_e2m1(packed):
    """Inverse of pack_e2m1: [..., K/2] bytes -> [..., K] 4-bit codes."""
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
