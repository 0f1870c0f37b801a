#!/usr/bin/env python3
"""Throughput benchmark of the block-scaled quantized linear layer on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic,
seeded input, all inputs resident in HBM before the timed region:

  * fp8r linear, 4096 tokens, K = 3072, N = 3072 (1 % outlier input channels):
    per-row E4M3 activation quantization + FP8 GEMM with row-wise scales;
  * nvfp4 linear, 4096 tokens, K = 3072, N = 12288 (MLP-up shape):
    runtime nvfp4 activation quantization with the calibrated input_scale +
    W4A4 GEMM on decoded operands;
  * the fallback path: dequantization of both weight matrices to bf16.

Weights are generated in bf16 and quantized (and their global scale
calibrated) by the library itself before timing. `value` is the step's GEMM
work (2 M N K for both GEMMs) divided by the step time. The dominant kernel's
roofline entry uses per-launch durations measured with HIP events on the
launch stream; its HBM traffic comes from the rocprofv3 counter summary in
profiles/ when that summary was taken on the current kernel source.

Prints exactly one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOP/s + % MFMA peak for nvfp4/fp8r GEMM at M=4096,K=3072; HBM GB/s"
PEAK_F16_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 MFMA
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
M, K, N_FP8, N_FP4 = 4096, 3072, 3072, 12288
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_w4a4_4096x12288x3072_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def warm_gpu(fn, ms=60.0):
    """Call fn back to back until at least `ms` of GPU time has passed: the clocks need tens of
    milliseconds of sustained load to settle, and the GPU idles while inputs are generated."""
    import torch

    done, n = 0.0, 4
    while done < ms:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        done += e0.elapsed_time(e1)
        n *= 2


_SPACER = {}


def queue_ahead(ms=1.5):
    """Give the GPU about `ms` of work right before a timed region, so that every timed launch is
    already queued when the GPU reaches it: the events then time the GPU rather than the rate at
    which Python issues launches (a launch through ctypes costs several microseconds of host time,
    as much as the few-token kernels timed here). The work is a bf16 matmul. Used only for short,
    memory-bound kernels: the matmul leaves the clocks where a power-hungry GEMM runs them, which
    slowed a following fp8 GEMM of 38 us by a fifth."""
    import torch

    if "n" not in _SPACER:
        g = torch.Generator(device="cuda")
        g.manual_seed(3)
        a = torch.randn((4096, 4096), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        b = torch.randn((4096, 4096), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        c = torch.empty((4096, 4096), device="cuda", dtype=torch.bfloat16)
        mm = lambda: torch.matmul(a, b, out=c)
        warm_gpu(mm, ms=20.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(8):
            mm()
        e1.record()
        torch.cuda.synchronize()
        _SPACER["mm"] = mm
        _SPACER["n"] = max(1, int(ms / (e0.elapsed_time(e1) / 8)) + 1)
    for _ in range(_SPACER["n"]):
        _SPACER["mm"]()


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter summary, if current."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    from block_scaled_precision_row_amd import traffic
    if t.get("source_sha256") != traffic.source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(rows=64, reps=2):
    """The CPU oracle on a bounded sample of the same step: `rows` tokens of each linear.

    Per repetition the oracle quantizes the sampled activations, dequantizes
    both weight matrices (exact values and the bf16 fallback copies) and forms
    the fp64 products. The value is the sampled GEMM work (2 rows N K summed
    over both linears) per second, in TFLOP/s.
    """
    import numpy as np
    from threadpoolctl import threadpool_info

    from block_scaled_precision_row_amd import synthetic as syn
    from oracle import dequant, gemm, quant

    x2 = syn.activations(syn.FP8R_4096, M, K)[:rows]
    x3 = syn.activations(syn.NVFP4_UP, M, K)[:rows]
    w2 = syn.weights(syn.FP8R_4096, N_FP8, K)
    w3 = syn.weights(syn.NVFP4_UP, N_FP4, K)
    w2q, w2s = quant.quantize_fp8r(w2)
    g3 = quant.calibrate_global_scale(w3)
    w3q, w3s = quant.quantize_nvfp4(w3, g3)
    gx3 = quant.calibrate_global_scale(syn.activations(syn.NVFP4_UP, M, K))
    t0 = time.perf_counter()
    for _ in range(reps):
        xq, sx = quant.quantize_fp8r(x2)
        gemm.gemm_fp8r(xq, sx, w2q, w2s)
        xq3, sx3 = quant.quantize_nvfp4(x3, gx3)
        gemm.gemm_nvfp4(xq3, sx3, gx3, w3q, w3s, g3)
        dequant.dequant_fp8r_bf16(w2q, w2s)
        dequant.dequant_nvfp4_bf16(w3q, w3s, g3)
    dt = (time.perf_counter() - t0) / reps
    flops = 2.0 * rows * K * (N_FP8 + N_FP4)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": "%d of %d tokens of both linears per step (weights dequantized in full), %d steps, %.2f s/step"
                      % (rows, M, reps, dt),
            "cores_note": "cores = BLAS threads of the fp64 products (the quantizers and dequantization are "
                          "single-threaded NumPy)",
            "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(), "affinity_cpus": affinity}


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where unavailable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def quantized_output_comparison(L, dev, y3, y2, gemm3_args, gemm2_args, operands3, operands2, x3):
    """Linears feeding another quantized linear, in both producers and both output formats: the
    GEMM followed by the activation quantizer over its bf16 Y, against the GEMM that encodes Y
    itself (nvfp4 in its epilogue; fp8r from per-segment row maxima written by the epilogue and
    one encoding pass), with and without writing the bf16 Y. Ten back-to-back repetitions each
    after warming, us per linear; the codes are bit-identical (GPU tests)."""
    import torch

    lib = L.lib
    stream = torch.cuda.current_stream().cuda_stream
    P = lambda t: t.data_ptr()
    x3q, x3s, gx3, w3q, w3s, g3 = operands3
    x2q, x2s, w2q, w2s = operands2
    fp8, nv = L.BSQ_FMT_FP8R, L.BSQ_FMT_NVFP4

    def ws(fmt, Mo, No, with_y):
        n = lib.bsq_gemm_quantize_y_workspace_bytes(fmt, Mo, No, 1 if with_y else 0)
        return torch.empty((max(n, 256),), dtype=torch.uint8, device=dev), n

    def time_calls(calls):
        for fn, a in calls:
            st = fn(*a)
            if st != 0:
                raise L.BsqError(fn.__name__, st)
        warm_gpu(lambda: [fn(*a) for fn, a in calls])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            for fn, a in calls:
                fn(*a)
        e1.record()
        torch.cuda.synchronize()
        return round(e0.elapsed_time(e1) / 10 * 1e3, 2)

    out = {}
    # nvfp4 W4A4 linear 4096 x 12288 x 3072 as the producer
    gy3 = L.bsq_calibrate_global_scale(y3)
    q4 = torch.empty((M, N_FP4 // 2), dtype=torch.uint8, device=dev)
    s4 = torch.empty((M, N_FP4 // 16), dtype=torch.uint8, device=dev)
    q8 = torch.empty((M, N_FP4), dtype=torch.uint8, device=dev)
    d8 = torch.empty((M,), dtype=torch.float32, device=dev)
    w3 = (P(x3q), P(x3s), P(gx3), P(w3q), P(w3s), P(g3))
    wsy, nwsy = ws(fp8, M, N_FP4, True)
    wsn, nwsn = ws(fp8, M, N_FP4, False)
    out["w4a4_4096x12288x3072"] = {
        "to_nvfp4": {
            "gemm_then_quantizer": time_calls([
                (lib.bsq_gemm_nvfp4_q, gemm3_args),
                (lib.bsq_quantize_act_nvfp4, (P(y3), M, N_FP4, N_FP4, P(gy3), P(q4), P(s4), stream))]),
            "fused_no_bf16_y": time_calls([(lib.bsq_gemm_nvfp4_q_quantize_y, w3 + (
                P(gy3), P(q4), P(s4), None, 0, M, N_FP4, K, None, 0, stream))]),
            "fused_with_bf16_y": time_calls([(lib.bsq_gemm_nvfp4_q_quantize_y, w3 + (
                P(gy3), P(q4), P(s4), P(y3), N_FP4, M, N_FP4, K, None, 0, stream))]),
        },
        "to_fp8r": {
            "gemm_then_quantizer": time_calls([
                (lib.bsq_gemm_nvfp4_q, gemm3_args),
                (lib.bsq_quantize_act_fp8r, (P(y3), M, N_FP4, N_FP4, P(q8), P(d8), stream))]),
            "fused_no_bf16_y": time_calls([(lib.bsq_gemm_nvfp4_q_quantize_y_fp8r, w3 + (
                P(q8), P(d8), None, 0, M, N_FP4, K, P(wsn), nwsn, stream))]),
            "fused_with_bf16_y": time_calls([(lib.bsq_gemm_nvfp4_q_quantize_y_fp8r, w3 + (
                P(q8), P(d8), P(y3), N_FP4, M, N_FP4, K, P(wsy), nwsy, stream))]),
        },
    }
    # fp8r W8A8 linear 4096 x 3072 x 3072 as the producer
    gy2 = L.bsq_calibrate_global_scale(y2)
    q4 = torch.empty((M, N_FP8 // 2), dtype=torch.uint8, device=dev)
    s4 = torch.empty((M, N_FP8 // 16), dtype=torch.uint8, device=dev)
    q8 = torch.empty((M, N_FP8), dtype=torch.uint8, device=dev)
    d8 = torch.empty((M,), dtype=torch.float32, device=dev)
    w2 = (P(x2q), P(x2s), P(w2q), P(w2s))
    entry = {}
    for name, fmt in (("to_nvfp4", nv), ("to_fp8r", fp8)):
        qq, qs = (q4, s4) if fmt == nv else (q8, d8)
        gy = P(gy2) if fmt == nv else None
        quantizer = ((lib.bsq_quantize_act_nvfp4, (P(y2), M, N_FP8, N_FP8, P(gy2), P(q4), P(s4), stream)) if fmt == nv
                     else (lib.bsq_quantize_act_fp8r, (P(y2), M, N_FP8, N_FP8, P(q8), P(d8), stream)))
        wy, nwy = ws(fmt, M, N_FP8, True)
        wn, nwn = ws(fmt, M, N_FP8, False)
        entry[name] = {
            "gemm_then_quantizer": time_calls([(lib.bsq_gemm_fp8r_q, gemm2_args), quantizer]),
            "fused_no_bf16_y": time_calls([(lib.bsq_gemm_fp8r_q_quantize_y, w2 + (
                fmt, gy, P(qq), P(qs), None, 0, M, N_FP8, K, P(wn), nwn, stream))]),
            "fused_with_bf16_y": time_calls([(lib.bsq_gemm_fp8r_q_quantize_y, w2 + (
                fmt, gy, P(qq), P(qs), P(y2), N_FP8, M, N_FP8, K, P(wy), nwy, stream))]),
        }
    out["fp8r_4096x3072x3072"] = entry
    # weight-only W4A16 linear 4096 x 12288 x 3072 (bf16 X) as the producer
    q4 = torch.empty((M, N_FP4 // 2), dtype=torch.uint8, device=dev)
    s4 = torch.empty((M, N_FP4 // 16), dtype=torch.uint8, device=dev)
    q8 = torch.empty((M, N_FP4), dtype=torch.uint8, device=dev)
    d8 = torch.empty((M,), dtype=torch.float32, device=dev)
    wo_gemm = (lib.bsq_gemm_nvfp4, (P(x3), K, P(w3q), P(w3s), P(g3), None, P(y3), N_FP4, M, N_FP4, K,
                                    L.BSQ_WEIGHT_ONLY, None, 0, stream))
    entry = {}
    for name, fmt in (("to_nvfp4", nv), ("to_fp8r", fp8)):
        qq, qs = (q4, s4) if fmt == nv else (q8, d8)
        gy = P(gy3) if fmt == nv else None
        quantizer = ((lib.bsq_quantize_act_nvfp4, (P(y3), M, N_FP4, N_FP4, P(gy3), P(q4), P(s4), stream)) if fmt == nv
                     else (lib.bsq_quantize_act_fp8r, (P(y3), M, N_FP4, N_FP4, P(q8), P(d8), stream)))
        wy, nwy = ws(fmt, M, N_FP4, True)
        wn, nwn = ws(fmt, M, N_FP4, False)
        fused = lambda y, ldy, wsp, nws: (lib.bsq_gemm_weight_only_quantize_y, (
            nv, P(x3), K, P(w3q), P(w3s), P(g3), fmt, gy, P(qq), P(qs), y, ldy, M, N_FP4, K, wsp, nws, stream))
        entry[name] = {
            "gemm_then_quantizer": time_calls([wo_gemm, quantizer]),
            "fused_no_bf16_y": time_calls([fused(None, 0, P(wn), nwn)]),
            "fused_with_bf16_y": time_calls([fused(P(y3), N_FP4, P(wy), nwy)]),
        }
    out["w4a16_4096x12288x3072"] = entry
    out["note"] = ("us per linear (GEMM on pre-quantized activations, or for the W4A16 producer on bf16 "
                   "activations, + the next linear's input encoding); fused = the producer encodes its own "
                   "output (nvfp4 in the epilogue, fp8r from the epilogue's per-segment row maxima and one "
                   "encoding pass)")
    return out


def lora_overhead(L, syn, dev, x2, x3, w2q, w2s, w3q, w3s, g3, gx3, reps=10):
    """LoRA side path: each linear from bf16 X (activation quantization + GEMM) without and with a
    synthetic adapter of several ranks (down projection + GEMM with the up projection fused),
    warm, in us: medians of 20 alternating pairs of calls; plus the down projection alone (mean
    of `reps` back-to-back calls) and its rate over the bytes it must move (X read once, A read,
    T written). Also a 16-token nvfp4 linear, whose short calls are queued behind other GPU work
    (queue_ahead) so that the host's launch cost is not timed."""
    import torch

    lib = L.lib
    stream = torch.cuda.current_stream().cuda_stream
    P = lambda t: t.data_ptr()

    def up_bf16(bits):
        return torch.from_numpy(bits.view("int16")).to(dev).view(torch.bfloat16)

    def paired(plain, call, pairs=20, ahead=False):
        """median us per call of the plain linear and of the linear with the adapter, timed in
        alternating pairs (each call between two events on the stream), so that clock and
        power drift affect both alike"""
        for fn, a in (plain, call):
            st = fn(*a)
            if st != 0:
                raise L.BsqError(fn.__name__, st)
        warm_gpu(lambda: (plain[0](*plain[1]), call[0](*call[1])))
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(pairs)]
        if ahead:
            queue_ahead()
        for e in ev:
            e[0].record()
            plain[0](*plain[1])
            e[1].record()
            call[0](*call[1])
            e[2].record()
        torch.cuda.synchronize()
        tp = sorted(e[0].elapsed_time(e[1]) * 1e3 for e in ev)
        tl = sorted(e[1].elapsed_time(e[2]) * 1e3 for e in ev)
        return tp[pairs // 2], tl[pairs // 2]

    def timed(fn, a, ahead=False):
        st = fn(*a)
        if st != 0:
            raise L.BsqError(fn.__name__, st)
        warm_gpu(lambda: fn(*a), ms=20.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if ahead:
            queue_ahead()
        e0.record()
        for _ in range(reps):
            fn(*a)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    out = {}
    layers = [("nvfp4", "nvfp4_4096x12288x3072", x3, M, N_FP4), ("fp8r", "fp8r_4096x3072x3072", x2, M, N_FP8),
              ("nvfp4", "nvfp4_16x12288x3072", x3[:16], 16, N_FP4)]
    for scheme, name, x, Mx, N in layers:
        fmt = L.BSQ_FMT_NVFP4 if scheme == "nvfp4" else L.BSQ_FMT_FP8R
        y = torch.empty((Mx, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty((lib.bsq_lora_workspace_bytes(fmt, Mx, N, K, 128, 0),), dtype=torch.uint8, device=dev)
        if scheme == "nvfp4":
            plain = (lib.bsq_gemm_nvfp4, (P(x), K, P(w3q), P(w3s), P(g3), P(gx3), P(y), N, Mx, N, K, 0, P(ws),
                                          ws.numel(), stream))
        else:
            plain = (lib.bsq_gemm_fp8r, (P(x), K, P(w2q), P(w2s), P(y), N, Mx, N, K, 0, P(ws), ws.numel(), stream))
        entry = {"ranks": {}}
        for rank in (16, 32, 64, 128):
            a, b = syn.lora_adapter(syn.NVFP4_UP if scheme == "nvfp4" else syn.FP8R_4096, rank, N, K)
            da, db = up_bf16(a), up_bf16(b)
            if scheme == "nvfp4":
                call = (lib.bsq_gemm_nvfp4_lora, (P(x), K, P(w3q), P(w3s), P(g3), P(gx3), P(da), P(db), rank, 1.0,
                                                  P(y), N, Mx, N, K, 0, P(ws), ws.numel(), stream))
            else:
                call = (lib.bsq_gemm_fp8r_lora, (P(x), K, P(w2q), P(w2s), P(da), P(db), rank, 1.0, P(y), N, Mx, N,
                                                 K, 0, P(ws), ws.numel(), stream))
            plain_us, us = paired(plain, call, ahead=Mx <= 64)
            t = torch.empty((Mx, rank), dtype=torch.bfloat16, device=dev)
            dws = torch.empty((max(1, lib.bsq_lora_down_workspace_bytes(Mx, K, rank)),), dtype=torch.uint8,
                              device=dev)
            # two short launches per call: queued behind GPU work at every size, so that the
            # events time the GPU rather than the host's launch rate
            down_us = timed(lib.bsq_lora_down, (P(x), K, P(da), Mx, K, rank, 1.0, P(t), P(dws), dws.numel(), stream),
                            ahead=True)
            down_bytes = Mx * K * 2 + rank * K * 2 + Mx * rank * 2
            entry["ranks"][str(rank)] = {
                "plain_us": round(plain_us, 2), "us": round(us, 2),
                "overhead_pct": round(100.0 * (us / plain_us - 1.0), 2), "down_us": round(down_us, 2),
                "down_gbs": round(down_bytes / (down_us * 1e-6) / 1e9, 1)}
        out[name] = entry
    out["note"] = ("whole linear from bf16 X in both columns (activation quantizer + GEMM; with the adapter also "
                   "its down projection), synthetic adapter with scale 1; the pages report about 5 % more "
                   "generation time with a LoRA attached (whole model, other hardware). down_us: the down "
                   "projection alone (bsq_lora_down); in the linears it is fused with the activation "
                   "encoding (whole-row kernel up to K = 6144 at these row counts, K-sliced kernel where the "
                   "routing prefers it, e.g. the 16-token linear)")
    return out


def vendor_gemm_context(dev, reps=20):
    """Context, not part of the path: the ROCm vendor library's GEMMs (hipBLASLt, through
    torch.matmul in bf16 and torch._scaled_mm with row-wise fp32 scales in E4M3) on the two step
    shapes with random operands, warmed like everything else; us per call (mean of `reps`)."""
    import torch

    out = {}

    def t(fn):
        warm_gpu(fn)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    g = torch.Generator(device=dev)
    g.manual_seed(11)
    for Mv, Nv, Kv in ((M, N_FP4, K), (M, N_FP8, K)):
        x = torch.randn((Mv, Kv), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        w = (torch.randn((Nv, Kv), generator=g, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
        wt = w.t().contiguous()
        name = "%dx%dx%d" % (Mv, Nv, Kv)
        us = t(lambda: torch.matmul(x, wt))
        out["bf16_matmul_" + name] = {"us": round(us, 1), "tflops": round(2.0 * Mv * Nv * Kv / us / 1e6, 1)}
        try:
            xf, wf = x.to(torch.float8_e4m3fn), w.to(torch.float8_e4m3fn)
            sa = torch.ones((Mv, 1), device=dev)
            sb = torch.ones((1, Nv), device=dev)
            us = t(lambda: torch._scaled_mm(xf, wf.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16))
            out["fp8_rowwise_scaled_mm_" + name] = {"us": round(us, 1),
                                                    "tflops": round(2.0 * Mv * Nv * Kv / us / 1e6, 1)}
        except (RuntimeError, TypeError) as e:
            out["fp8_rowwise_scaled_mm_" + name] = "unavailable: %s" % str(e)[:80]
        del x, w, wt
    out["note"] = "vendor library on plain bf16 / E4M3 operands, for context only (not the nvfp4 path)"
    return out


def small_m_sweep(L, syn, dev, Ms=(16, 32, 64, 128, 256, 512), Ns=(N_FP8, N_FP4)):
    """Few-token GEMMs (K = 3072), all four schemes, with cold weights.

    Each configuration is launched 24 times back to back between two events, rotating over
    enough weight copies (> 600 MB) that no launch finds its weights in the 256 MB Infinity
    Cache; activations are pre-quantized for W4A4 / W8A8 (the quantizer is timed separately).
    Bytes are the algorithmic ones: weights + activations + Y.
    """
    import torch

    lib = L.lib
    stream = torch.cuda.current_stream().cuda_stream
    P = lambda t: t.data_ptr()

    def up_bf16(bits):
        return torch.from_numpy(bits.view("int16")).to(dev).view(torch.bfloat16)

    def timed(calls, iters=24, warm=3):
        it = iter(range(1 << 30))
        warm_gpu(lambda: calls[next(it) % len(calls)](), ms=30.0)
        for i in range(warm):
            calls[i % len(calls)]()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        queue_ahead()
        e0.record()
        for i in range(iters):
            calls[i % len(calls)]()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters * 1e3  # us

    def check(st):
        if st != 0:
            raise L.BsqError("small-M sweep", st)

    rows = []
    for N in Ns:
        w = up_bf16(syn.weights(syn.SMALL_M, N, K))
        gw = L.bsq_calibrate_global_scale(w)
        wp, ws = L.bsq_quantize_act_nvfp4(w, gw)
        wq, sw = L.bsq_quantize_act_fp8r(w)
        del w
        r4 = int(600e6 // (wp.numel() + ws.numel())) + 1
        r8 = int(600e6 // wq.numel()) + 1
        W4 = [(wp.clone(), ws.clone()) for _ in range(r4)]
        W8 = [(wq.clone(), sw.clone()) for _ in range(r8)]
        for Mi in Ms:
            x = up_bf16(syn.activations(syn.SMALL_M, Mi, K))
            gx = L.bsq_calibrate_global_scale(x)
            xq8, sx8 = L.bsq_quantize_act_fp8r(x)
            xq4, sx4 = L.bsq_quantize_act_nvfp4(x, gx)
            y = torch.empty((Mi, N), dtype=torch.bfloat16, device=dev)
            us = {
                "w4a4": timed([lambda i=i: check(lib.bsq_gemm_nvfp4_q(P(xq4), P(sx4), P(gx), P(W4[i][0]), P(W4[i][1]),
                                                                      P(gw), P(y), N, Mi, N, K, stream))
                               for i in range(r4)]),
                "w4a16": timed([lambda i=i: check(lib.bsq_gemm_nvfp4(P(x), K, P(W4[i][0]), P(W4[i][1]), P(gw), None,
                                                                     P(y), N, Mi, N, K, L.BSQ_WEIGHT_ONLY, None, 0,
                                                                     stream))
                                for i in range(r4)]),
                "w8a8": timed([lambda i=i: check(lib.bsq_gemm_fp8r_q(P(xq8), P(sx8), P(W8[i][0]), P(W8[i][1]), P(y),
                                                                     N, Mi, N, K, stream))
                               for i in range(r8)]),
                "w8a16": timed([lambda i=i: check(lib.bsq_gemm_fp8r(P(x), K, P(W8[i][0]), P(W8[i][1]), P(y), N, Mi,
                                                                    N, K, L.BSQ_WEIGHT_ONLY, None, 0, stream))
                                for i in range(r8)]),
            }
            nbytes = {
                "w4a4": N * K // 2 + N * K // 16 + Mi * K // 2 + Mi * K // 16 + 2 * Mi * N,
                "w4a16": N * K // 2 + N * K // 16 + 2 * Mi * K + 2 * Mi * N,
                "w8a8": N * K + 4 * N + Mi * K + 4 * Mi + 2 * Mi * N,
                "w8a16": N * K + 4 * N + 2 * Mi * K + 2 * Mi * N,
            }
            rows.append({"M": Mi, "N": N, "us": {k: round(v, 2) for k, v in us.items()},
                         "hbm_frac": {k: round(nbytes[k] / (us[k] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4) for k in us},
                         "tflops": {k: round(2.0 * Mi * N * K / (us[k] * 1e-6) / 1e12, 1) for k in us}})
            log("small-M M=%d N=%d: %s" % (Mi, N, rows[-1]["us"]))
        del W4, W8
        torch.cuda.empty_cache()
    return {"K": K, "cold": True, "rows": rows,
            "note": "kernel time per call from events around 24 back-to-back launches (weights rotated over > 600 MB), "
                    "queued behind ~1.5 ms of other GPU work so that host launch cost is not timed; "
                    "hbm_frac = (weights + activations + Y bytes) / time / 8 TB/s"}


def block_launches(L, syn, dev, Ms=(1, 16, 32, 512, 2048)):
    """A joint block's four linears (qkv 9216x3072, proj 3072x3072, up 12288x3072, down 3072x12288) with
    cold weights: four launches back to back against one grouped launch (bsq_gemm_grouped_q), per
    scheme and token count. At 1, 16 and 32 tokens the group runs as one grid of the few-token kernels,
    at 512 tokens as one grid of 128 x 128 tiles two to a compute unit, at 2048 tokens as one grid of
    256 x 192 tiles.

    The block's weights are copied until the copies exceed 600 MB and the timed calls rotate over
    them, so that no call finds its weights in the 256 MB Infinity Cache; activations are
    pre-quantized. Bytes per block are the algorithmic ones: weights + activations + Y.
    """
    import torch

    lib = L.lib
    stream = torch.cuda.current_stream().cuda_stream
    P = lambda t: t.data_ptr()

    def up_bf16(bits):
        return torch.from_numpy(bits.view("int16")).to(dev).view(torch.bfloat16)

    def check(st):
        if st != 0:
            raise L.BsqError("block launches", st)

    def timed(calls, iters=24):
        it = iter(range(1 << 30))
        warm_gpu(lambda: calls[next(it) % len(calls)](), ms=30.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        queue_ahead()
        e0.record()
        for i in range(iters):
            calls[i % len(calls)]()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters * 1e3  # us per block

    gemms = syn.JOINT_GEMMS
    out = {"gemms": [{"gemm": n, "N": N, "K": K} for n, N, K in gemms], "rows": [], "weight_only_rows": []}
    for scheme in ("nvfp4", "fp8r"):
        block = []
        for gi, (name, N, K) in enumerate(gemms):
            w = up_bf16(syn.weights(syn.JOINT_4MP, N, K, block=gi))
            if scheme == "nvfp4":
                gw = L.bsq_calibrate_global_scale(w)
                block.append((*L.bsq_quantize_act_nvfp4(w, gw), gw))
            else:
                block.append(L.bsq_quantize_act_fp8r(w))
            del w
        wbytes = sum(sum(t.numel() * t.element_size() for t in b) for b in block)
        copies = [block] + [[tuple(t.clone() for t in b) for b in block] for _ in range(int(600e6 // wbytes))]
        for Mi in Ms:
            xs = {}
            for K in sorted({K for _, _, K in gemms}):
                x = up_bf16(syn.activations(syn.JOINT_4MP, Mi, K, block=0 if K == 3072 else 1))
                if scheme == "nvfp4":
                    gx = L.bsq_calibrate_global_scale(x)
                    xs[K] = (*L.bsq_quantize_act_nvfp4(x, gx), gx)
                else:
                    xs[K] = L.bsq_quantize_act_fp8r(x)
            ys = [torch.empty((Mi, N), dtype=torch.bfloat16, device=dev) for _, N, _ in gemms]
            singles, groups = [], []
            for cp in copies:
                probs = (L.GemmProblem * len(gemms))()
                one = []
                for gi, (name, N, K) in enumerate(gemms):
                    xa, w, y = xs[K], cp[gi], ys[gi]
                    if scheme == "nvfp4":
                        probs[gi] = L.GemmProblem(P(xa[0]), P(xa[1]), P(xa[2]), P(w[0]), P(w[1]), P(w[2]), P(y), N, Mi,
                                                  N, K)
                        one.append(lambda xa=xa, w=w, y=y, N=N, K=K: check(lib.bsq_gemm_nvfp4_q(
                            P(xa[0]), P(xa[1]), P(xa[2]), P(w[0]), P(w[1]), P(w[2]), P(y), N, Mi, N, K, stream)))
                    else:
                        probs[gi] = L.GemmProblem(P(xa[0]), P(xa[1]), None, P(w[0]), P(w[1]), None, P(y), N, Mi, N,
                                                  K)
                        one.append(lambda xa=xa, w=w, y=y, N=N, K=K: check(lib.bsq_gemm_fp8r_q(
                            P(xa[0]), P(xa[1]), P(w[0]), P(w[1]), P(y), N, Mi, N, K, stream)))
                singles.append(lambda one=one: [c() for c in one])
                fmt = L.BSQ_FMT_NVFP4 if scheme == "nvfp4" else L.BSQ_FMT_FP8R
                groups.append(lambda probs=probs, fmt=fmt: check(lib.bsq_gemm_grouped_q(fmt, probs, len(gemms),
                                                                                         stream)))
            us_four, us_grouped = timed(singles), timed(groups)
            nbytes = wbytes + sum(xs[K][0].numel() + xs[K][1].numel() * xs[K][1].element_size() for K in xs) \
                + sum(2 * Mi * N for _, N, _ in gemms)
            row = {"scheme": scheme, "M": Mi, "four_launches_us": round(us_four, 2),
                   "grouped_us": round(us_grouped, 2),
                   "hbm_frac_four_launches": round(nbytes / (us_four * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                   "hbm_frac_grouped": round(nbytes / (us_grouped * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                   "block_mb": round(nbytes / 1e6, 2)}
            out["rows"].append(row)
            log("joint block %s M=%d: four launches %.1f us, one grouped launch %.1f us" %
                (scheme, Mi, us_four, us_grouped))
            del ys, singles, groups
        # the same weights as weight-only linears (bf16 activations): bsq_gemm_grouped_weight_only
        for Mi in (1, 16):
            xb = {K: up_bf16(syn.activations(syn.JOINT_4MP, Mi, K, block=0 if K == 3072 else 1))
                  for K in sorted({K for _, _, K in gemms})}
            ys = [torch.empty((Mi, N), dtype=torch.bfloat16, device=dev) for _, N, _ in gemms]
            singles, groups = [], []
            fmt = L.BSQ_FMT_NVFP4 if scheme == "nvfp4" else L.BSQ_FMT_FP8R
            for cp in copies:
                probs = (L.WeightOnlyProblem * len(gemms))()
                one = []
                for gi, (name, N, K) in enumerate(gemms):
                    x, w, y = xb[K], cp[gi], ys[gi]
                    if scheme == "nvfp4":
                        probs[gi] = L.WeightOnlyProblem(P(x), K, P(w[0]), P(w[1]), P(w[2]), P(y), N, Mi, N, K)
                        one.append(lambda x=x, w=w, y=y, N=N, K=K: check(lib.bsq_gemm_nvfp4(
                            P(x), K, P(w[0]), P(w[1]), P(w[2]), None, P(y), N, Mi, N, K, L.BSQ_WEIGHT_ONLY, None, 0,
                            stream)))
                    else:
                        probs[gi] = L.WeightOnlyProblem(P(x), K, P(w[0]), P(w[1]), None, P(y), N, Mi, N, K)
                        one.append(lambda x=x, w=w, y=y, N=N, K=K: check(lib.bsq_gemm_fp8r(
                            P(x), K, P(w[0]), P(w[1]), P(y), N, Mi, N, K, L.BSQ_WEIGHT_ONLY, None, 0, stream)))
                singles.append(lambda one=one: [c() for c in one])
                groups.append(lambda probs=probs, fmt=fmt: check(lib.bsq_gemm_grouped_weight_only(
                    fmt, probs, len(gemms), stream)))
            us_four, us_grouped = timed(singles), timed(groups)
            out["weight_only_rows"].append({"scheme": scheme, "M": Mi, "four_launches_us": round(us_four, 2),
                                            "grouped_us": round(us_grouped, 2)})
            log("weight-only joint block %s M=%d: four launches %.1f us, one grouped launch %.1f us" %
                (scheme, Mi, us_four, us_grouped))
            del ys, singles, groups
        del copies, block
        torch.cuda.empty_cache()
    out["note"] = ("us per block (the four GEMMs) from events around 24 back-to-back blocks rotated over > 600 MB of "
                   "weight copies (cold weights), queued behind other GPU work; hbm_frac = (weights + activations + "
                   "Y bytes) / time / 8 TB/s; weight_only_rows: the same weights as weight-only linears (bf16 "
                   "activations, bsq_gemm_grouped_weight_only)")
    return out


def joint_block_sweep(L, syn, dev, reps=5):
    """The 4-megapixel joint-block workload: 16384 tokens through the four linears of a block
    (qkv 9216x3072, proj 3072x3072, up 12288x3072, down 3072x12288), once as an nvfp4 W4A4 block
    and once as an fp8r W8A8 block (the 28 blocks alternate the two schemes).

    Weights follow the synthetic recipe (blocks 0 and 1); the two activation tensors
    ([16384, 3072] and [16384, 12288], N(0, 1)) are drawn on the GPU with a fixed seed for speed.
    Activations are quantized once per scheme outside the timing; each GEMM is timed over `reps`
    back-to-back launches. `gemm_ms_28_blocks` = 14 x (nvfp4 block) + 14 x (fp8r block).
    """
    import torch

    lib = L.lib
    stream = torch.cuda.current_stream().cuda_stream
    P = lambda t: t.data_ptr()
    Mj = syn.JOINT_TOKENS
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    xs = {k: torch.randn((Mj, k), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
          for k in sorted({kk for _, _, kk in syn.JOINT_GEMMS})}

    def timed(fn):
        warm_gpu(fn)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3  # us

    def check(st):
        if st != 0:
            raise L.BsqError("joint-block sweep", st)

    out = {"tokens": Mj, "gemms": []}
    block_us = {"nvfp4": 0.0, "fp8r": 0.0}
    seq_us, grouped_us = {}, {}
    quant_us = {"nvfp4": 0.0, "fp8r": 0.0}
    for scheme, block in (("nvfp4", 0), ("fp8r", 1)):
        xq = {}
        for k, x in xs.items():
            if scheme == "nvfp4":
                gx = L.bsq_calibrate_global_scale(x)
                q, sq = L.bsq_quantize_act_nvfp4(x, gx)
                xq[k] = (q, sq, gx)
                quant_us[scheme] += timed(lambda: check(lib.bsq_quantize_act_nvfp4(P(x), Mj, k, k, P(gx), P(q), P(sq),
                                                                                    stream)))
            else:
                q, sq = L.bsq_quantize_act_fp8r(x)
                xq[k] = (q, sq, None)
                quant_us[scheme] += timed(lambda: check(lib.bsq_quantize_act_fp8r(P(x), Mj, k, k, P(q), P(sq), stream)))
        calls, keep = [], []
        probs = (L.GemmProblem * len(syn.JOINT_GEMMS))()
        for gi, (name, N, Kj) in enumerate(syn.JOINT_GEMMS):
            w = torch.from_numpy(syn.weights(syn.JOINT_4MP, N, Kj, block=block * 4 + gi).view("int16")) \
                .to(dev).view(torch.bfloat16)
            y = torch.empty((Mj, N), dtype=torch.bfloat16, device=dev)
            q, sq, gx = xq[Kj]
            if scheme == "nvfp4":
                gw = L.bsq_calibrate_global_scale(w)
                wq, ws = L.bsq_quantize_act_nvfp4(w, gw)
                call = (lambda q=q, sq=sq, gx=gx, wq=wq, ws=ws, gw=gw, y=y, N=N, Kj=Kj:
                        check(lib.bsq_gemm_nvfp4_q(P(q), P(sq), P(gx), P(wq), P(ws), P(gw), P(y), N, Mj, N, Kj,
                                                   stream)))
                probs[gi] = L.GemmProblem(P(q), P(sq), P(gx), P(wq), P(ws), P(gw), P(y), N, Mj, N, Kj)
                keep += [wq, ws, gw, y]
                peak = PEAK_F16_TFLOPS
            else:
                wq, ws = L.bsq_quantize_act_fp8r(w)
                call = (lambda q=q, sq=sq, wq=wq, ws=ws, y=y, N=N, Kj=Kj:
                        check(lib.bsq_gemm_fp8r_q(P(q), P(sq), P(wq), P(ws), P(y), N, Mj, N, Kj, stream)))
                probs[gi] = L.GemmProblem(P(q), P(sq), None, P(wq), P(ws), None, P(y), N, Mj, N, Kj)
                keep += [wq, ws, y]
                peak = PEAK_FP8_TFLOPS
            us = timed(call)
            calls.append(call)
            tf = 2.0 * Mj * N * Kj / (us * 1e-6) / 1e12
            out["gemms"].append({"scheme": scheme, "gemm": name, "N": N, "K": Kj, "us": round(us, 1),
                                 "tflops": round(tf, 1), "frac_peak": round(tf / peak, 4)})
            block_us[scheme] += us
            log("joint block %s %s %dx%dx%d: %.1f us, %.0f TFLOP/s" % (scheme, name, Mj, N, Kj, us, tf))
            del w
        # the whole block: its four launches back to back, against one grouped launch of all four
        fmt = L.BSQ_FMT_NVFP4 if scheme == "nvfp4" else L.BSQ_FMT_FP8R
        seq_us[scheme] = timed(lambda: [c() for c in calls])
        grouped_us[scheme] = timed(lambda: check(lib.bsq_gemm_grouped_q(fmt, probs, len(calls), stream)))
        log("joint block %s: four launches %.1f us, one grouped launch %.1f us"
            % (scheme, seq_us[scheme], grouped_us[scheme]))
        del calls, keep, probs
    out["block_us"] = {k: round(v, 1) for k, v in block_us.items()}
    out["activation_quant_us_per_block"] = {k: round(v, 1) for k, v in quant_us.items()}
    out["gemm_ms_28_blocks"] = round(14 * (block_us["nvfp4"] + block_us["fp8r"]) / 1e3, 2)
    out["block_us_four_launches"] = {k: round(v, 1) for k, v in seq_us.items()}
    out["block_us_grouped"] = {k: round(v, 1) for k, v in grouped_us.items()}
    out["gemm_ms_28_blocks_grouped"] = round(14 * (grouped_us["nvfp4"] + grouped_us["fp8r"]) / 1e3, 2)
    out["frac_of_ideal_28_blocks_grouped"] = round(
        28 * 2.0 * Mj * sum(N * K for _, N, K in syn.JOINT_GEMMS) / 2 * (1 / PEAK_F16_TFLOPS + 1 / PEAK_FP8_TFLOPS)
        / 1e9 / out["gemm_ms_28_blocks_grouped"], 4)
    out["note"] = ("peaks: f16 MFMA for nvfp4 (decoded operands), fp8 MFMA for fp8r; activations pre-quantized "
                   "(their quantization time per block listed separately); gemm_ms_28_blocks sums the GEMMs timed "
                   "one by one, gemm_ms_28_blocks_grouped times each block's four GEMMs as one grouped launch "
                   "(bsq_gemm_grouped_q); frac_of_ideal = the 28 blocks' flops at the f16 (nvfp4) and fp8 (fp8r) "
                   "MFMA peaks over the grouped time")
    del xs
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU needs 30-50 ms of sustained load to reach its steady clocks (a W4A4 GEMM measured
    # 430 us on the first call, 280 us after 7 ms, 236 us from 50 ms on): the default warmup is
    # about 0.2 s of steps, so that the timed steps see the steady state
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=600)
    ap.add_argument("--warm-ms", type=float, default=100.0,
                    help="GPU time of back-to-back steps run after the warmup steps and before the timed ones, "
                         "whatever --warmup says, so that the timed steps see steady clocks")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    ap.add_argument("--no-small-m", action="store_true", help="skip the few-token sweep")
    ap.add_argument("--no-joint", action="store_true", help="skip the 16384-token joint-block shapes")
    ap.add_argument("--no-quant-out", action="store_true", help="skip the quantized-output comparison")
    ap.add_argument("--no-lora", action="store_true", help="skip the LoRA side-path measurement")
    ap.add_argument("--no-vendor", action="store_true", help="skip the vendor-library GEMM context")
    ap.add_argument("--only-step", action="store_true",
                    help="time the step only (no CPU baseline, no extra measurements), e.g. under a profiler")
    args = ap.parse_args()
    if args.only_step:
        args.no_cpu_baseline = args.no_small_m = args.no_joint = args.no_quant_out = args.no_lora = True
        args.no_vendor = True
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path (requested %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    from block_scaled_precision_row_amd import _lib as L
    from block_scaled_precision_row_amd import synthetic as syn

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up_bf16(bits):
        return torch.from_numpy(bits.view("int16")).to(dev).view(torch.bfloat16)

    log("generating inputs")
    x2 = up_bf16(syn.activations(syn.FP8R_4096, M, K))
    x3 = up_bf16(syn.activations(syn.NVFP4_UP, M, K))
    w2 = up_bf16(syn.weights(syn.FP8R_4096, N_FP8, K))
    w3 = up_bf16(syn.weights(syn.NVFP4_UP, N_FP4, K))
    # weights to their storage formats, global scales calibrated, by the library
    w2q, w2s = L.bsq_quantize_act_fp8r(w2)
    g3 = L.bsq_calibrate_global_scale(w3)
    w3q, w3s = L.bsq_quantize_act_nvfp4(w3, g3)
    gx3 = L.bsq_calibrate_global_scale(x3)
    del w2, w3
    x2q = torch.empty((M, K), dtype=torch.uint8, device=dev)
    x2s = torch.empty((M,), dtype=torch.float32, device=dev)
    x3q = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    x3s = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    y2 = torch.empty((M, N_FP8), dtype=torch.bfloat16, device=dev)
    y3 = torch.empty((M, N_FP4), dtype=torch.bfloat16, device=dev)
    wd2 = torch.empty((N_FP8, K), dtype=torch.bfloat16, device=dev)
    wd3 = torch.empty((N_FP4, K), dtype=torch.bfloat16, device=dev)

    # the timed loop calls the C entry points directly (argument tuples built once) so that host
    # overhead stays far below the GPU time of a step
    P = lambda t: t.data_ptr()
    lib = L.lib
    parts = ["quant_fp8r", "gemm_fp8r", "quant_nvfp4", "gemm_nvfp4", "dequant_fp8r", "dequant_nvfp4"]

    def calls(stream):
        return [
            (lib.bsq_quantize_act_fp8r, (P(x2), M, K, K, P(x2q), P(x2s), stream)),
            (lib.bsq_gemm_fp8r_q, (P(x2q), P(x2s), P(w2q), P(w2s), P(y2), N_FP8, M, N_FP8, K, stream)),
            (lib.bsq_quantize_act_nvfp4, (P(x3), M, K, K, P(gx3), P(x3q), P(x3s), stream)),
            (lib.bsq_gemm_nvfp4_q, (P(x3q), P(x3s), P(gx3), P(w3q), P(w3s), P(g3), P(y3), N_FP4, M, N_FP4, K, stream)),
            (lib.bsq_dequant_to_bf16, (L.BSQ_FMT_FP8R, P(w2q), P(w2s), None, N_FP8, K, P(wd2), stream)),
            (lib.bsq_dequant_to_bf16, (L.BSQ_FMT_NVFP4, P(w3q), P(w3s), P(g3), N_FP4, K, P(wd3), stream)),
        ]
    stream = torch.cuda.current_stream().cuda_stream
    seq = calls(stream)
    DOM = parts.index("gemm_nvfp4")
    FP8 = parts.index("gemm_fp8r")

    def step(ev=None):
        for i, (fn, a) in enumerate(seq):
            if ev is not None and i in (DOM, FP8):
                ev[0 if i == DOM else 2].record()
            st = fn(*a)
            if st != 0:
                raise L.BsqError(fn.__name__, st)
            if ev is not None and i in (DOM, FP8):
                ev[1 if i == DOM else 3].record()

    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # then at least --warm-ms of back-to-back steps, timed by events: the clocks need tens of
    # milliseconds of sustained load to settle, whatever the number of warmup steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    warm_gpu(step, ms=args.warm_ms)
    e1.record()
    torch.cuda.synchronize()
    warm_ms = e0.elapsed_time(e1)
    log("warmed for %.1f ms of steps" % warm_ms)

    log("timing %d steps" % args.steps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    fp8_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / args.steps

    # per-kernel averages (outside the timed region): each call back to back between two events
    per_kernel = {}
    for i, p in enumerate(parts):
        fn, a = seq[i]
        reps = 5 if i == DOM else 40
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn(*a)
        e0.record()
        for _ in range(reps):
            fn(*a)
        e1.record()
        torch.cuda.synchronize()
        per_kernel[p] = e0.elapsed_time(e1) / reps  # ms
    b2b = {"gemm_nvfp4": per_kernel["gemm_nvfp4"], "gemm_fp8r": per_kernel["gemm_fp8r"]}
    per_kernel["gemm_nvfp4"] = dom_ms
    per_kernel["gemm_fp8r"] = fp8_ms
    ms_per_step = wall * 1e3 / args.steps
    flops = 2.0 * M * K * (N_FP8 + N_FP4)
    value = flops * args.steps / wall / 1e12

    g4_us = per_kernel["gemm_nvfp4"] * 1e3
    g4_tflops = 2.0 * M * N_FP4 * K / (g4_us * 1e-6) / 1e12
    g8_us = per_kernel["gemm_fp8r"] * 1e3
    g8_tflops = 2.0 * M * N_FP8 * K / (g8_us * 1e-6) / 1e12

    def gbs(nbytes, ms):
        return nbytes / (ms * 1e-3) / 1e9

    hbm = {
        "quant_fp8r": gbs(M * K * 2 + M * K + 4 * M, per_kernel["quant_fp8r"]),
        "quant_nvfp4": gbs(M * K * 2 + M * K // 2 + M * K // 16, per_kernel["quant_nvfp4"]),
        "dequant_fp8r": gbs(N_FP8 * K + 4 * N_FP8 + N_FP8 * K * 2, per_kernel["dequant_fp8r"]),
        "dequant_nvfp4": gbs(N_FP4 * K // 2 + N_FP4 * K // 16 + 4 + N_FP4 * K * 2, per_kernel["dequant_nvfp4"]),
    }

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_gpu_ms": round(warm_ms, 1),
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8,f16",
        "data": "synthetic",
        "config": {
            "workload": "fp8r W8A8 linear 4096x3072x3072 (1% outlier channels) + nvfp4 W4A4 linear "
                        "4096x12288x3072 (MLP-up) + bf16 dequant fallback of both weights, one GPU",
            "tokens": M, "K": K, "N_fp8r": N_FP8, "N_nvfp4": N_FP4,
        },
        "roofline": {
            "kernel": "gemm_w4a4 (nvfp4 W4A4 GEMM, 4096x12288x3072, f16 MFMA on decoded operands)",
            "bound": "mfma",
            "achieved": round(g4_tflops, 1),
            "peak": PEAK_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(g4_tflops / PEAK_F16_TFLOPS, 4),
            "traffic": measured_traffic(),
        },
        "kernels_us": {p: round(v * 1e3, 2) for p, v in per_kernel.items()},
        "kernels_us_note": "gemm_nvfp4, gemm_fp8r: HIP events around each launch in the timed steps (on the "
                           "launch stream); others: back-to-back launches between two events after the timed region",
        "gemm_fp8r": {"tflops": round(g8_tflops, 1), "frac_fp8_peak": round(g8_tflops / PEAK_FP8_TFLOPS, 4),
                      "back_to_back_us": round(b2b["gemm_fp8r"] * 1e3, 2),
                      "frac_fp8_peak_back_to_back": round(2.0 * M * N_FP8 * K / (b2b["gemm_fp8r"] * 1e-3) / 1e12
                                                          / PEAK_FP8_TFLOPS, 4)},
        "gemm_nvfp4": {"tflops": round(g4_tflops, 1), "frac_f16_peak": round(g4_tflops / PEAK_F16_TFLOPS, 4),
                       "frac_fp4_peak": round(g4_tflops / 10100.0, 4),
                       "back_to_back_us": round(b2b["gemm_nvfp4"] * 1e3, 2),
                       "frac_f16_peak_back_to_back": round(2.0 * M * N_FP4 * K / (b2b["gemm_nvfp4"] * 1e-3) / 1e12
                                                           / PEAK_F16_TFLOPS, 4)},
        "gemm_note": "tflops / frac from the in-step events (each launch's pair also holds its dispatch latency, "
                     "about 3 us); back_to_back: 40 (fp8r) or 5 (nvfp4) launches queued between two events after "
                     "the timed region, closer to the kernel's own duration",
        "hbm_gbs": {k: round(v, 1) for k, v in hbm.items()},
        "hbm_frac": {k: round(v / PEAK_HBM_GBS, 4) for k, v in hbm.items()},
    }
    if not args.no_quant_out:
        log("quantized-output comparison")
        result["quantized_output_us"] = quantized_output_comparison(
            L, dev, y3, y2, seq[DOM][1], seq[FP8][1], (x3q, x3s, gx3, w3q, w3s, g3), (x2q, x2s, w2q, w2s), x3)
    if not args.no_vendor:
        log("vendor-library GEMM context")
        result["vendor_gemm_context"] = vendor_gemm_context(dev)
    if not args.no_lora:
        log("LoRA side path")
        result["lora"] = lora_overhead(L, syn, dev, x2, x3, w2q, w2s, w3q, w3s, g3, gx3)
    if not args.no_small_m:
        log("few-token sweep")
        result["small_m"] = small_m_sweep(L, syn, dev)
    if not args.no_small_m:
        log("joint block: four launches vs one grouped launch")
        result["block_launches"] = block_launches(L, syn, dev)
    if not args.no_joint:
        log("joint-block shapes")
        result["joint_block_4mp"] = joint_block_sweep(L, syn, dev)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline()
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
