"""Helpers shared by the GPU parity tests: device upload / download and the
GEMM tolerance.

Tolerance for bf16 GEMM outputs (fp32 accumulation, bf16 rounding of Y):
both must hold
  normwise   ||Y_gpu - Y_ref||_F / ||Y_ref||_F <= 1e-2
  elementwise |y_gpu - y_ref| <= 1e-2 |y_ref| + 1e-3 rms(Y_ref)
where Y_ref is the oracle's fp64 product of the exactly dequantized
operands. The floor term covers outputs near zero under cancellation; the
expected error is about 2^-9 normwise from the bf16 output rounding.
A path that rounds an intermediate as well (the LoRA side path holds its
rank-r product T in bf16) adds that rounding's own elementwise bound.
"""
import numpy as np
import torch

REL_TOL = 1e-2
FLOOR = 1e-3


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev(arr):
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def dev_scalar(v):
    return torch.tensor([float(np.float32(v))], dtype=torch.float32, device="cuda")


def host(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gemm_errors(y_gpu_bits, y_ref, extra=None):
    y = bf16_to_f64(y_gpu_bits)
    diff = np.abs(y - y_ref)
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    norm = float(np.linalg.norm(y - y_ref) / max(np.linalg.norm(y_ref), 1e-300))
    allow = REL_TOL * np.abs(y_ref) + FLOOR * rms + (0.0 if extra is None else extra)
    excess = float(np.max(diff - allow)) if y_ref.size else -1.0
    return norm, excess, float(diff.max()) if diff.size else 0.0, rms


def assert_gemm_close(y_gpu_bits, y_ref, what="", extra=None):
    """``extra``: an optional elementwise allowance added to the bound, for a stated
    intermediate rounding on top of the output's."""
    norm, excess, maxdiff, rms = gemm_errors(y_gpu_bits, y_ref, extra)
    print("%s normwise=%.3e maxabs=%.3e rms=%.3e" % (what, norm, maxdiff, rms), flush=True)
    assert np.all(np.isfinite(bf16_to_f64(y_gpu_bits))), what
    assert norm <= REL_TOL, (what, norm)
    assert excess <= 0.0, (what, excess)


def assert_gemm_close_by_row(y_gpu_bits, y_ref, what=""):
    """The tolerance applied to each row on its own (the floor from that row's rms): for inputs
    whose rows differ in magnitude by many binades, where one rms over the whole output would
    hide the small rows. A row whose reference is all zero must come out all zero."""
    y = bf16_to_f64(y_gpu_bits)
    assert np.all(np.isfinite(y)), what
    worst = 0.0
    for m in range(y_ref.shape[0]):
        r, g = y_ref[m], y[m]
        rms = float(np.sqrt(np.mean(r ** 2)))
        if rms == 0.0:
            assert np.all(g == 0.0), (what, m)
            continue
        norm = float(np.linalg.norm(g - r) / np.linalg.norm(r))
        assert norm <= REL_TOL, (what, m, norm)
        assert np.all(np.abs(g - r) <= REL_TOL * np.abs(r) + FLOOR * rms), (what, m)
        worst = max(worst, norm)
    print("%s worst row normwise=%.3e" % (what, worst), flush=True)
