"""GPU parity: quantizers, calibration and bf16 dequantization against the oracle.

All of these are bit-exact: codes, block scales, row scales, global scales
and dequantized bf16 weights must equal the oracle's bytes on the same
seeded inputs. Calls go through the C ABI via the ctypes binding.
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_row_amd import synthetic as syn
from oracle import codec, dequant, quant
from tests.gpu_util import dev, dev_bf16, dev_scalar, host

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from block_scaled_precision_row_amd import _lib as L


def bf16(v):
    return codec.f32_to_bf16(np.asarray(v, np.float64))


def _all_bf16_up_to(limit):
    b = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        v = (b << 16).view(np.float32).astype(np.float64)
    keep = np.isfinite(v) & (np.abs(v) <= limit)
    return b[keep].astype(np.uint16)


def _varied_rows(M, K, seed):
    """Rows of normals with per-row magnitudes spread over 2^-40 .. 2^40, some zero rows and blocks."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((M, K)) * 2.0 ** rng.integers(-40, 40, size=(M, 1))
    z[rng.random((M, K)) < 0.02] = 0.0
    z[::17] = 0.0
    z[min(3, M - 1), ::2] = -0.0
    z[min(5, M - 1), :16] = 0.0
    return bf16(z)


def _check_fp8r(x_bits, ldx_pad=0):
    M, K = x_bits.shape
    qr, dr = quant.quantize_fp8r(x_bits)
    if ldx_pad:
        xp = np.zeros((M, K + ldx_pad), np.uint16)
        xp[:, :K] = x_bits
        xd = dev_bf16(xp)[:, :K]
    else:
        xd = dev_bf16(x_bits)
    q, d = L.bsq_quantize_act_fp8r(xd)
    torch.cuda.synchronize()
    assert np.array_equal(host(q), qr), "fp8r codes differ"
    assert np.array_equal(host(d).view(np.uint32), dr.view(np.uint32)), "fp8r row scales differ"


def _check_nvfp4(x_bits, g, ldx_pad=0):
    M, K = x_bits.shape
    pr, sr = quant.quantize_nvfp4(x_bits, g)
    if ldx_pad:
        xp = np.zeros((M, K + ldx_pad), np.uint16)
        xp[:, :K] = x_bits
        xd = dev_bf16(xp)[:, :K]
    else:
        xd = dev_bf16(x_bits)
    p, s = L.bsq_quantize_act_nvfp4(xd, dev_scalar(g))
    torch.cuda.synchronize()
    assert np.array_equal(host(s), sr), "nvfp4 block scales differ"
    assert np.array_equal(host(p), pr), "nvfp4 codes differ"


def test_fp8r_every_bf16_value_at_unit_scale():
    vals = _all_bf16_up_to(448.0)
    K = 4096
    n_rows = -(-len(vals) // (K - 1))
    x = np.zeros((n_rows, K), np.uint16)
    flat = np.zeros(n_rows * (K - 1), np.uint16)
    flat[:len(vals)] = vals
    x[:, 1:] = flat.reshape(n_rows, K - 1)
    x[:, 0] = bf16([448.0])[0]                    # d = 1, r = 1
    _check_fp8r(x)


@pytest.mark.parametrize("M,K,pad", [(77, 96, 0), (5, 32, 8), (64, 4096, 0), (9, 8192, 24), (3, 16384, 0), (2, 20480, 8)])
def test_fp8r_varied_rows(M, K, pad):
    _check_fp8r(_varied_rows(M, K, M * 7 + K), pad)


def test_fp8r_benchmark_shapes():
    _check_fp8r(syn.activations(syn.FP8R_4096, 4096, 3072))
    _check_fp8r(syn.weights(syn.FP8R_4096, 3072, 3072))
    _check_fp8r(syn.activations(syn.JOINT_4MP, 512, 12288, block=1))


def test_nvfp4_every_bf16_value_at_unit_scale():
    vals = _all_bf16_up_to(6.0)
    per_block = 15
    nblk = -(-len(vals) // per_block)
    blocks = np.zeros((nblk, 16), np.uint16)
    flat = np.zeros(nblk * per_block, np.uint16)
    flat[:len(vals)] = vals
    blocks[:, 1:] = flat.reshape(nblk, per_block)
    blocks[:, 0] = bf16([6.0])[0]                  # block max 6 -> scale 1, r = 1
    nb_row = 16
    nrow = -(-nblk // nb_row)
    allb = np.zeros((nrow * nb_row, 16), np.uint16)
    allb[:nblk] = blocks
    _check_nvfp4(allb.reshape(nrow, nb_row * 16), np.float32(1.0))


@pytest.mark.parametrize("M,K,pad,g", [(77, 96, 0, 0.0123), (5, 32, 8, 1.0), (64, 4096, 0, 3e-5),
                                        (9, 8192, 24, 2.0 ** -20), (33, 256, 0, 7.5e8)])
def test_nvfp4_varied_rows(M, K, pad, g):
    _check_nvfp4(_varied_rows(M, K, M * 11 + K), np.float32(g), pad)


def test_nvfp4_benchmark_shapes():
    x = syn.activations(syn.NVFP4_UP, 4096, 3072)
    _check_nvfp4(x, quant.calibrate_global_scale(x))
    w = syn.weights(syn.NVFP4_UP, 12288, 3072)
    _check_nvfp4(w, quant.calibrate_global_scale(w))
    # beyond the calibrated range: saturating scales and codes
    _check_nvfp4(x, np.float32(quant.calibrate_global_scale(x) / 64))


@pytest.mark.parametrize("shape,seed", [((64, 256), 1), ((4096, 3072), 2), ((12288, 3072), 3), ((3, 32), 4)])
def test_calibrate_global_scale(shape, seed):
    x = syn.normal_bf16(shape, 99, seed, sigma=0.02 if seed % 2 else 1.0)
    gr = quant.calibrate_global_scale(x)
    g = L.bsq_calibrate_global_scale(dev_bf16(x))
    torch.cuda.synchronize()
    assert host(g).view(np.uint32)[0] == np.float32(gr).view(np.uint32)
    z = L.bsq_calibrate_global_scale(dev_bf16(np.zeros((5, 64), np.uint16)))
    assert float(host(z)[0]) == 1.0


@pytest.mark.parametrize("K", [3072, 2080])
def test_calibration_sees_every_chunk(K):
    """The tensor maximum planted in each of the reduction's per-lane streams (four interleaved
    8-value chunk streams and the row remainder) and in the last row: found every time."""
    M = 7
    base = syn.normal_bf16((M, K), 98, K, sigma=0.02)
    for row, col in ((0, 0), (1, 8 * 64 + 3), (2, 8 * 128 + 5), (3, 8 * 192 + 7), (4, 8 * 256 + 1), (5, K - 1),
                     (M - 1, K // 2)):
        x = base.copy()
        x[row, col] = np.uint16(0xC2F6)  # bf16 -123.0
        g = L.bsq_calibrate_global_scale(dev_bf16(x))
        torch.cuda.synchronize()
        assert host(g).view(np.uint32)[0] == np.float32(quant.calibrate_global_scale(x)).view(np.uint32), (row, col)
        assert abs(float(host(g)[0]) * 2688.0 - 123.0) < 1e-3


@pytest.mark.parametrize("N,K", [(3072, 3072), (12288, 3072), (77, 96), (1, 32)])
def test_dequant_bf16_bitexact(N, K):
    w = syn.normal_bf16((N, K), syn.SMALL_M, 10 + N % 7, sigma=0.02)
    g = quant.calibrate_global_scale(w)
    p, s = quant.quantize_nvfp4(w, g)
    ref = dequant.dequant_nvfp4_bf16(p, s, g)
    out = L.bsq_dequant_to_bf16(L.BSQ_FMT_NVFP4, dev(p), dev(s), dev_scalar(g))
    torch.cuda.synchronize()
    assert np.array_equal(host(out), ref), "nvfp4 dequant differs"
    q, d = quant.quantize_fp8r(w)
    ref8 = dequant.dequant_fp8r_bf16(q, d)
    out8 = L.bsq_dequant_to_bf16(L.BSQ_FMT_FP8R, dev(q), dev(d))
    torch.cuda.synchronize()
    assert np.array_equal(host(out8), ref8), "fp8r dequant differs"


def test_dequant_every_code_and_scale():
    """All 256 packed bytes under every finite positive E4M3 block scale; all E4M3 codes under varied row scales."""
    sfs = np.arange(1, 0x7F, dtype=np.uint8)                    # 126 block scales
    N, K = len(sfs), 512                                         # 512 values = 256 bytes = 32 blocks per row
    p = np.tile(np.arange(256, dtype=np.uint8), (N, 1))
    s = np.repeat(sfs[:, None], K // 16, axis=1)
    for g in (np.float32(1.0), np.float32(3.3e-3), np.float32(1e30)):
        ref = dequant.dequant_nvfp4_bf16(p, s, g)
        out = L.bsq_dequant_to_bf16(L.BSQ_FMT_NVFP4, dev(p), dev(s), dev_scalar(g))
        torch.cuda.synchronize()
        assert np.array_equal(host(out), ref)
    codes = np.tile(np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8), (5, 1))
    codes = np.concatenate([codes, codes[:, :2]], axis=1)[:, :256]
    d = np.array([1.0, 2.0 ** -20, 0.37, 1e10, 0.0], np.float32)
    ref8 = dequant.dequant_fp8r_bf16(codes, d)
    out8 = L.bsq_dequant_to_bf16(L.BSQ_FMT_FP8R, dev(codes), dev(d))
    torch.cuda.synchronize()
    assert np.array_equal(host(out8), ref8)


def test_quantizers_deterministic():
    x = dev_bf16(syn.activations(syn.FP8R_4096, 1024, 3072))
    a = [host(t).copy() for t in L.bsq_quantize_act_fp8r(x)]
    b = [host(t).copy() for t in L.bsq_quantize_act_fp8r(x)]
    assert all(np.array_equal(u, v) for u, v in zip(a, b))
