"""Oracle dequantization: exact dequantized values and the bf16 fallback weights.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The fallback ("BFL (fp8r / nvfp4)", last paragraph of the "Kernels" section)
dequantizes the stored weights to the compute dtype (bf16) and runs a plain
linear. Rounding order taken for the bf16 weights:

    nvfp4: w = bf16(rn32(p * g)) with p = e2m1(q) * e4m3(sf) exact (<= 6 significant bits)
    fp8r:  w = bf16(rn32(e4m3(q) * d_n))

The exact values (``*_values``) are the real numbers the codes stand for; they
are what the GEMM reference multiplies.
"""

import numpy as np

from .codec import e2m1_decode, e4m3_decode, f32_to_bf16, rn32, unpack_e2m1
from .quant import NVFP4_BLOCK


def nvfp4_values(packed, sf, g):
    """Exact real values e2m1 * e4m3(sf) * g, float64 [R, K]."""
    v = e2m1_decode(unpack_e2m1(packed))
    s = np.repeat(e4m3_decode(sf), NVFP4_BLOCK, axis=-1)
    return v * s * np.float64(np.float32(g))


def fp8r_values(codes, d):
    """Exact real values e4m3(q) * d_row, float64 [R, K]."""
    return e4m3_decode(codes) * np.asarray(d, dtype=np.float32).astype(np.float64)[..., None]


def dequant_nvfp4_bf16(packed, sf, g):
    """bf16 bit patterns of bf16(rn32(e2m1 * e4m3(sf) * g))."""
    v = e2m1_decode(unpack_e2m1(packed))
    p = v * np.repeat(e4m3_decode(sf), NVFP4_BLOCK, axis=-1)  # exact
    return f32_to_bf16(rn32(p * np.float64(np.float32(g))))


def dequant_fp8r_bf16(codes, d):
    """bf16 bit patterns of bf16(rn32(e4m3(q) * d_row))."""
    return f32_to_bf16(rn32(fp8r_values(codes, d)))
