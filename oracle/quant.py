"""Oracle quantizers: fp8r per-row E4M3 and nvfp4 E2M1 with E4M3 scales per 16.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Inputs are bf16 bit patterns (uint16). Every step written ``rn32(...)`` is one
correctly rounded fp32 operation on fp32 operands; maxima and the bf16 -> fp32
widening are exact.

fp8r ("BFL (fp8r / nvfp4)", fp8r bullet: E4M3 weight with an fp32 scale per
row; activations quantized to E4M3 per row at run time). The per-row scale
maps the row's largest magnitude onto the E4M3 maximum 448:

    a = max_k |x_k|,  d = rn32(a / 448),  r = rn32(1 / d),
    q_k = E4M3(rn32(x_k * r)),  stored scale d,  dequant e4m3(q) * d.

A row of zeros stores d = 0 and signed-zero codes. For weights the "row" is
an output channel (one scale per row of W[N, K]); for activations it is a
token (one per row of X[M, K]).

nvfp4 (same page, nvfp4 bullet: packed E2M1, E4M3 block scales over 16, fp32
global ``weight_scale_2``, calibrated fp32 ``input_scale``). The block scale
maps the block's largest magnitude onto the E2M1 maximum 6 after the global
scale g is divided out:

    G = rn32(1 / g)                                   (once per tensor)
    a_b = max_{k in b} |x_k|                          (16-element block b)
    sf_b = E4M3(rn32(rn32(a_b / 6) * G))
    r_b = 0 if sf_b == 0 else rn32(G / e4m3(sf_b))
    q_k = E2M1(rn32(x_k * r_b))                       dequant e2m1(q) * e4m3(sf_b) * g

Calibration: g = rn32(amax / (6 * 448)) over the whole tensor, i.e. the
tensor maximum lands on the largest representable product 6 * 448. A tensor
of zeros is given g = 1 (any positive value quantizes it to zeros).
Activations beyond the calibrated range saturate (sf at 448, codes at +-6).
"""

import numpy as np

from .codec import (E2M1_MAX, E4M3_MAX, bf16_to_f64, e4m3_decode, encode_e2m1,
                    encode_e4m3, pack_e2m1, rn32)

NVFP4_BLOCK = 16


def quantize_fp8r(x_bits):
    """bf16 [R, K] -> (E4M3 codes uint8 [R, K], per-row fp32 scale d as float32 [R])."""
    x = bf16_to_f64(x_bits)
    a = np.max(np.abs(x), axis=-1) if x.shape[-1] else np.zeros(x.shape[:-1])
    d = rn32(a / E4M3_MAX)
    with np.errstate(divide="ignore"):
        r = np.where(d > 0, rn32(1.0 / np.where(d > 0, d, 1.0)), 0.0)
    v = rn32(x * r[..., None])
    return encode_e4m3(v), d.astype(np.float32)


def calibrate_global_scale(x_bits):
    """Global nvfp4 scale for a bf16 tensor: rn32(amax / 2688), or 1 for an all-zero tensor."""
    x = bf16_to_f64(x_bits)
    a = float(np.max(np.abs(x))) if x.size else 0.0
    if a == 0.0:
        return np.float32(1.0)
    return np.float32(rn32(a / (E2M1_MAX * E4M3_MAX)))


def nvfp4_block_scales(x_bits, g):
    """Per-16 block scales: (sf codes uint8 [R, K/16], encode multipliers r_b float64 [R, K/16])."""
    x = bf16_to_f64(x_bits)
    R, K = x.shape
    assert K % NVFP4_BLOCK == 0
    G = rn32(1.0 / np.float64(np.float32(g)))
    a = np.abs(x.reshape(R, K // NVFP4_BLOCK, NVFP4_BLOCK)).max(axis=-1) if K else np.zeros((R, 0))
    sf = encode_e4m3(rn32(rn32(a / E2M1_MAX) * G))
    sfv = e4m3_decode(sf)
    with np.errstate(divide="ignore"):
        r = np.where(sfv > 0, rn32(G / np.where(sfv > 0, sfv, 1.0)), 0.0)
    return sf, r


def quantize_nvfp4(x_bits, g):
    """bf16 [R, K] with global scale g -> (packed E2M1 uint8 [R, K/2], E4M3 block scales uint8 [R, K/16])."""
    x = bf16_to_f64(x_bits)
    R, K = x.shape
    sf, r = nvfp4_block_scales(x_bits, g)
    xb = x.reshape(R, K // NVFP4_BLOCK, NVFP4_BLOCK)
    v = rn32(xb * r[..., None])
    codes = encode_e2m1(v).reshape(R, K)
    return pack_e2m1(codes), sf
