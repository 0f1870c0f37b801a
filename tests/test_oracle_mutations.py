"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

Each case monkeypatches one oracle function with a subtly wrong variant and
runs a pin test, which must then fail. This shows the pins are strong enough
that such a mistake anywhere in the oracle would not go unnoticed.
"""
import numpy as np
import pytest

from oracle import codec, dequant, gemm, quant
from tests import test_oracle_codec as tc
from tests import test_oracle_gemm as tg
from tests import test_oracle_quant as tq


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_swapped_nibbles_caught(monkeypatch):
    def bad_pack(codes):
        c = np.asarray(codes).astype(np.uint8) & 0xF
        return (c[..., 1::2] | (c[..., 0::2] << 4)).astype(np.uint8)
    monkeypatch.setattr(codec, "pack_e2m1", bad_pack)
    _fails(tc.test_packing_fixture)


def test_round_half_away_caught(monkeypatch):
    real = codec.encode_e2m1
    def bad(v):
        v = np.asarray(v, np.float64)
        a = np.minimum(np.abs(v), 6.0)
        q = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
        mag = np.minimum(np.floor(a / q + 0.5) * q, 6.0)
        return real(np.where(np.signbit(v), -mag, mag))
    monkeypatch.setattr(codec, "encode_e2m1", bad)
    _fails(tc.test_rounding_at_every_midpoint_and_one_ulp_off, "e2m1")


def test_wrong_e4m3_bias_caught(monkeypatch):
    monkeypatch.setattr(codec, "E4M3_TABLE", codec.E4M3_TABLE * 2)
    _fails(tc.test_e4m3_anchors_match_fixture)


def test_block_scale_divides_by_wrong_max_caught(monkeypatch):
    monkeypatch.setattr(quant, "E2M1_MAX", 4.0)
    _fails(tq.test_nvfp4_worked_block)


def test_block_of_8_caught(monkeypatch):
    monkeypatch.setattr(quant, "NVFP4_BLOCK", 8)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        tq.test_nvfp4_block_max_lands_on_6_and_error_bound()


def test_missing_global_reciprocal_caught(monkeypatch):
    real_rn32 = quant.rn32

    def bad_scales(x_bits, g):
        x = codec.bf16_to_f64(x_bits)
        R, K = x.shape
        G = np.float64(np.float32(g))      # mistake: multiplies by g instead of 1/g
        a = np.abs(x.reshape(R, K // 16, 16)).max(axis=-1)
        sf = codec.encode_e4m3(real_rn32(real_rn32(a / 6.0) * G))
        sfv = codec.e4m3_decode(sf)
        r = np.where(sfv > 0, real_rn32(G / np.where(sfv > 0, sfv, 1.0)), 0.0)
        return sf, r
    monkeypatch.setattr(quant, "nvfp4_block_scales", bad_scales)
    _fails(tq.test_nvfp4_power_of_two_scales_reduce_to_plain_rounding, 2)


def test_dropped_global_scale_in_dequant_caught(monkeypatch):
    def bad(packed, sf, g):
        v = codec.e2m1_decode(codec.unpack_e2m1(packed))
        return v * np.repeat(codec.e4m3_decode(sf), 16, axis=-1)
    monkeypatch.setattr(dequant, "nvfp4_values", bad)
    _fails(tq.test_nvfp4_block_max_lands_on_6_and_error_bound)


def test_fp8r_scale_on_wrong_axis_caught(monkeypatch):
    def bad(codes, d):
        return codec.e4m3_decode(codes) * np.asarray(d, np.float32).astype(np.float64)[None, :]
    monkeypatch.setattr(dequant, "fp8r_values", bad)
    with pytest.raises((AssertionError, ValueError)):
        tq.test_fp8r_row_max_lands_on_448_and_error_bound()


def test_transposed_operand_caught(monkeypatch):
    monkeypatch.setattr(gemm, "matmul_nt", lambda a, b: np.asarray(a, np.float64) @ np.asarray(b, np.float64).T[::-1])
    _fails(tg.test_selection_matrix_returns_weight_columns)


def test_rowwise_fp8r_max_over_columns_caught(monkeypatch):
    def bad(x_bits):
        x = codec.bf16_to_f64(x_bits)
        a = np.max(np.abs(x), axis=0)[: x.shape[0]]      # mistake: max over the wrong axis
        a = np.resize(a, x.shape[0])
        d = codec.rn32(a / 448.0)
        r = np.where(d > 0, codec.rn32(1.0 / np.where(d > 0, d, 1.0)), 0.0)
        return codec.encode_e4m3(codec.rn32(x * r[:, None])), d.astype(np.float32)
    monkeypatch.setattr(quant, "quantize_fp8r", bad)
    _fails(tq.test_fp8r_row_max_lands_on_448_and_error_bound)


def test_lora_dropped_scale_caught(monkeypatch):
    from oracle import lora
    from tests import test_oracle_lora as tl
    monkeypatch.setattr(lora, "scale_f32", lambda s: np.float64(1.0))
    _fails(tl.test_delta_equals_exact_rank_one_sum, 3, 5, 32, 2)


def test_lora_up_projection_read_as_its_transpose_caught(monkeypatch):
    from oracle import codec as oc
    from oracle import lora
    from tests import test_oracle_lora as tl

    def bad(x_bits, a_bits, b_bits, scale):
        t = lora.lora_down(x_bits, a_bits, scale)
        bm = oc.bf16_to_f64(b_bits)
        return t @ bm.reshape(bm.shape[1], bm.shape[0])  # B's storage taken as [r][N]
    monkeypatch.setattr(lora, "lora_delta", bad)
    _fails(tl.test_merged_weight_identity)


def test_lora_down_projection_transposed_caught(monkeypatch):
    from oracle import codec as oc
    from oracle import lora
    from tests import test_oracle_lora as tl

    def bad(x_bits, a_bits, scale):
        am = oc.bf16_to_f64(a_bits)
        return lora.scale_f32(scale) * (oc.bf16_to_f64(x_bits) @ am.reshape(am.shape[1], am.shape[0]))
    monkeypatch.setattr(lora, "lora_down", bad)
    _fails(tl.test_merged_weight_identity)


# ---- operation order of the quantizers' fp32 steps ---------------------------------
# The pages fix the formats, not the order of the fp32 steps; these are the plausible
# other orders, each of which changes codes on scales that are not powers of two.

def test_fp8r_divides_by_row_scale_caught(monkeypatch):
    def bad(x_bits):
        x = codec.bf16_to_f64(x_bits)
        a = np.max(np.abs(x), axis=-1)
        d = codec.rn32(a / 448.0)
        v = codec.rn32(x / np.where(d > 0, d, 1.0)[..., None])   # mistake: x / d, not x * fp32(1/d)
        return codec.encode_e4m3(v), d.astype(np.float32)
    monkeypatch.setattr(quant, "quantize_fp8r", bad)
    _fails(tq.test_fp8r_worked_row_with_inexact_reciprocal)


def test_nvfp4_scale_from_one_division_caught(monkeypatch):
    def bad_scales(x_bits, g):
        x = codec.bf16_to_f64(x_bits)
        R, K = x.shape
        g64 = np.float64(np.float32(g))
        a = np.abs(x.reshape(R, K // 16, 16)).max(axis=-1)
        sf = codec.encode_e4m3(codec.rn32(a / (6.0 * g64)))        # mistake: a / (6 g) in one step
        sfv = codec.e4m3_decode(sf)
        G = codec.rn32(1.0 / g64)
        r = np.where(sfv > 0, codec.rn32(G / np.where(sfv > 0, sfv, 1.0)), 0.0)
        return sf, r
    monkeypatch.setattr(quant, "nvfp4_block_scales", bad_scales)
    _fails(tq.test_nvfp4_worked_blocks_with_inexact_global_reciprocal)


def test_nvfp4_multiplier_from_scale_times_global_caught(monkeypatch):
    real = quant.nvfp4_block_scales

    def bad_scales(x_bits, g):
        sf, _ = real(x_bits, g)
        sfv = codec.e4m3_decode(sf)
        sg = codec.rn32(sfv * np.float64(np.float32(g)))
        r = np.where(sfv > 0, codec.rn32(1.0 / np.where(sfv > 0, sg, 1.0)), 0.0)   # mistake: 1 / (sf g)
        return sf, r
    monkeypatch.setattr(quant, "nvfp4_block_scales", bad_scales)
    _fails(tq.test_nvfp4_worked_blocks_with_inexact_global_reciprocal)


def test_nvfp4_both_steps_by_division_caught(monkeypatch):
    def bad_scales(x_bits, g):
        x = codec.bf16_to_f64(x_bits)
        R, K = x.shape
        g64 = np.float64(np.float32(g))
        a = np.abs(x.reshape(R, K // 16, 16)).max(axis=-1)
        sf = codec.encode_e4m3(codec.rn32(a / (6.0 * g64)))
        sfv = codec.e4m3_decode(sf)
        r = np.where(sfv > 0, codec.rn32(1.0 / np.where(sfv > 0, sfv * g64, 1.0)), 0.0)
        return sf, r
    monkeypatch.setattr(quant, "nvfp4_block_scales", bad_scales)
    _fails(tq.test_nvfp4_worked_blocks_with_inexact_global_reciprocal)
