"""Oracle GEMMs: Y = X W^T in fp64 from exactly dequantized operands.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"BFL (fp8r / nvfp4)", "Kernels" section: fp8r runs an fp8 GEMM with row-wise
scales, nvfp4 quantizes the activations at run time and runs an fp4 GEMM, and
the fallback multiplies unquantized activations by dequantized weights. All
produce bf16 Y = X W^T (no bias). Every dequantized operand value is a dyadic
rational, so the exact product is well defined; ``exact_matmul`` computes it
with ``fractions.Fraction`` for tiny shapes, and the fp64 BLAS product is the
reference at full size (relative error ~K * 2^-53, far below the tolerance).
"""

from fractions import Fraction

import numpy as np

from .codec import bf16_to_f64
from .dequant import fp8r_values, nvfp4_values


def matmul_nt(a, b):
    """fp64 A[M, K] @ B[N, K]^T."""
    return np.asarray(a, np.float64) @ np.asarray(b, np.float64).T


def gemm_fp8r(xq, sx, wq, sw):
    """W8A8: (e4m3(xq) * sx[m]) (e4m3(wq) * sw[n])^T."""
    return matmul_nt(fp8r_values(xq, sx), fp8r_values(wq, sw))


def gemm_fp8r_weight_only(x_bits, wq, sw):
    """W8A16: bf16 X times exactly dequantized fp8r W."""
    return matmul_nt(bf16_to_f64(x_bits), fp8r_values(wq, sw))


def gemm_nvfp4(xq, sfx, gx, wq, sfw, gw):
    """W4A4: dequantized nvfp4 X times dequantized nvfp4 W."""
    return matmul_nt(nvfp4_values(xq, sfx, gx), nvfp4_values(wq, sfw, gw))


def gemm_nvfp4_weight_only(x_bits, wq, sfw, gw):
    """W4A16: bf16 X times exactly dequantized nvfp4 W."""
    return matmul_nt(bf16_to_f64(x_bits), nvfp4_values(wq, sfw, gw))


def linear_bf16(x_bits, w_bits):
    """Fallback linear: bf16 X times bf16 W (both exact), fp64."""
    return matmul_nt(bf16_to_f64(x_bits), bf16_to_f64(w_bits))


def exact_matmul(a, b):
    """Exact rational A[M, K] @ B[N, K]^T by a triple loop over Fractions (tiny shapes only)."""
    A = [[Fraction(float(v)) for v in row] for row in np.asarray(a, np.float64)]
    B = [[Fraction(float(v)) for v in row] for row in np.asarray(b, np.float64)]
    return [[sum((A[i][k] * B[j][k] for k in range(len(A[i]))), Fraction(0)) for j in range(len(B))]
            for i in range(len(A))]
