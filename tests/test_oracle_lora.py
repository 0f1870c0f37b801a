"""Pins for the LoRA oracle: exact rational sums, the merged-weight identity, closed forms.

The adapter's contribution s (X A^T) B^T is compared with a Fraction loop that
sums rank-1 terms in its own order on tiny shapes where M, N, K and r all
differ (a transposed operand changes the shape or the values); with the
merged-weight identity, which multiplies B A first; with a one-hot rank-1
adapter whose output is known in closed form; and with the zero adapter.
"""
from fractions import Fraction

import numpy as np
import pytest

from block_scaled_precision_row_amd import synthetic
from oracle import codec, gemm, lora


def bf16(v):
    return codec.f32_to_bf16(np.asarray(v, np.float64))


def _rel(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def _frac(bits):
    return [[Fraction(float(v)) for v in row] for row in codec.bf16_to_f64(bits)]


SHAPES = [(3, 5, 32, 2), (1, 7, 16, 3), (4, 2, 48, 1), (2, 3, 64, 5)]


@pytest.mark.parametrize("M,N,K,r", SHAPES)
def test_delta_equals_exact_rank_one_sum(M, N, K, r):
    rng = np.random.default_rng(1000 * M + 100 * N + K + r)
    x = bf16(rng.standard_normal((M, K)))
    a = bf16(rng.standard_normal((r, K)) / np.sqrt(K))
    b = bf16(rng.standard_normal((N, r)) * 0.1)
    s = 1.0 / 3.0  # not a power of two: its fp32 rounding shows
    X, A, B = _frac(x), _frac(a), _frac(b)
    S = Fraction(float(np.float32(s)))
    # sum over the rank of outer products u_j v_j^T, u_j = X a_j (a column of T), v_j = B[:, j]
    exact = [[Fraction(0)] * N for _ in range(M)]
    for j in range(r):
        u = [sum((X[m][k] * A[j][k] for k in range(K)), Fraction(0)) for m in range(M)]
        for m in range(M):
            for n in range(N):
                exact[m][n] += S * u[m] * B[n][j]
    got = lora.lora_delta(x, a, b, s)
    assert got.shape == (M, N)
    assert _rel(got, [[float(v) for v in row] for row in exact]) < 1e-12
    t = lora.lora_down(x, a, s)
    assert t.shape == (M, r)
    t_exact = [[float(S * sum((X[m][k] * A[j][k] for k in range(K)), Fraction(0))) for j in range(r)]
               for m in range(M)]
    assert _rel(t, t_exact) < 1e-12


def test_merged_weight_identity():
    """W x + s B (A x) equals (W + s B A) x: the adapter is a rank-r change of the weight."""
    M, N, K, r = 16, 40, 96, 8
    x = synthetic.activations(synthetic.TINY, M, K)
    w = synthetic.weights(synthetic.TINY, N, K)
    a, b = synthetic.lora_adapter(synthetic.TINY, r, N, K)
    s = 0.625
    y = lora.lora_linear(gemm.linear_bf16(x, w), x, a, b, s)
    merged = codec.bf16_to_f64(w) + s * (codec.bf16_to_f64(b) @ codec.bf16_to_f64(a))
    ref = codec.bf16_to_f64(x) @ merged.T
    assert _rel(y, ref) < 1e-12
    # the adapter is a visible share of the output at this scale, so a dropped term shows
    d = lora.lora_delta(x, a, b, s)
    assert 0.02 < np.linalg.norm(d) / np.linalg.norm(y) < 1.0


def test_one_hot_rank_one_closed_form():
    """A = e_k0 (one row), B = a column b: the contribution is s * x[:, k0] b^T exactly."""
    rng = np.random.default_rng(7)
    M, N, K, k0 = 5, 9, 64, 37
    x = bf16(rng.standard_normal((M, K)))
    a = np.zeros((1, K))
    a[0, k0] = 1.0
    bcol = bf16(rng.standard_normal((N, 1)))
    d = lora.lora_delta(x, bf16(a), bcol, 0.5)
    expect = 0.5 * np.outer(codec.bf16_to_f64(x)[:, k0], codec.bf16_to_f64(bcol)[:, 0])
    assert np.array_equal(d, expect)


def test_zero_adapter_leaves_base():
    M, N, K, r = 4, 6, 32, 4
    x = synthetic.activations(synthetic.TINY, M, K)
    a, b = synthetic.lora_adapter(synthetic.TINY, r, N, K)
    base = np.arange(M * N, dtype=np.float64).reshape(M, N) / 7
    assert np.array_equal(lora.lora_linear(base, x, a, np.zeros_like(b), 1.0), base)
    assert np.array_equal(lora.lora_linear(base, x, a, b, 0.0), base)


def test_scale_is_taken_in_fp32():
    assert lora.scale_f32(0.1) == np.float64(np.float32(0.1)) != 0.1
