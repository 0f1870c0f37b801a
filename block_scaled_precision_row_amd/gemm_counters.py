"""rocprofv3 hardware counters of the two headline GEMMs, for their roofline analysis.

Workload (`run`): the nvfp4 W4A4 GEMM 4096x12288x3072 and the fp8r W8A8 GEMM 4096x3072x3072 on
seeded synthetic inputs, each warmed for about 60 ms of GPU time and then launched five times.
Collect one counter set per rocprofv3 run (the hardware cannot take them all at once), from
any directory with the repository on the module path (cd /tmp && export TMPDIR=/tmp
PYTHONPATH=<repo>):

    rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES \\
        SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_ACTIVE_INST_ANY \\
        -d <d1> -o run --output-format csv -- python3 -m block_scaled_precision_row_amd.gemm_counters run
    rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_VMEM SQ_LDS_BANK_CONFLICT \\
        SQ_WAIT_INST_LDS SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_VMEM \\
        -d <d2> -o run --output-format csv -- python3 -m block_scaled_precision_row_amd.gemm_counters run

    python3 -m block_scaled_precision_row_amd.gemm_counters summarize <d1>/run_counter_collection.csv \\
        <d2>/run_counter_collection.csv

`summarize` averages each counter over the last five dispatches of each GEMM (the warm ones) and
prints a markdown table with the raw sums and the derived fractions. Units (rocprofv3 sums each
counter over every hardware instance): GRBM_GUI_ACTIVE counts the dispatch's clock cycles once
per XCD (8 of them); SQ_VALU_MFMA_BUSY_CYCLES and SQ_VALU_MFMA_COEXEC_CYCLES count cycles per
SIMD (1024 SIMDs); SQ_WAVE_CYCLES, SQ_ACTIVE_INST_* and SQ_WAIT_* count wave-cycles in
quad-cycles (4 cycles). (Check: the W4A4 dispatch issues 9437184 MFMAs of 32 busy cycles each,
which is what SQ_VALU_MFMA_BUSY_CYCLES reads.)
"""
import csv
import sys

M, K = 4096, 3072
N_FP4, N_FP8 = 12288, 3072
SIMDS = 1024
XCDS = 8
KERNELS = {"gemm_w4a4_kernel": ("nvfp4 W4A4 4096x12288x3072", 2.0 * M * N_FP4 * K),
           "gemm_fp8_kernel": ("fp8r W8A8 4096x3072x3072", 2.0 * M * N_FP8 * K)}


def run(reps=5, warm_ms=60.0):
    import torch

    from block_scaled_precision_row_amd import _lib as L
    from block_scaled_precision_row_amd import synthetic as syn

    dev = torch.device("cuda:0")
    up = lambda bits: torch.from_numpy(bits.view("int16")).to(dev).view(torch.bfloat16)
    x3 = up(syn.activations(syn.NVFP4_UP, M, K))
    w3 = up(syn.weights(syn.NVFP4_UP, N_FP4, K))
    g3 = L.bsq_calibrate_global_scale(w3)
    w3q, w3s = L.bsq_quantize_act_nvfp4(w3, g3)
    gx3 = L.bsq_calibrate_global_scale(x3)
    x3q, x3s = L.bsq_quantize_act_nvfp4(x3, gx3)
    y3 = torch.empty((M, N_FP4), dtype=torch.bfloat16, device=dev)
    x2 = up(syn.activations(syn.FP8R_4096, M, K))
    w2 = up(syn.weights(syn.FP8R_4096, N_FP8, K))
    w2q, w2s = L.bsq_quantize_act_fp8r(w2)
    x2q, x2s = L.bsq_quantize_act_fp8r(x2)
    y2 = torch.empty((M, N_FP8), dtype=torch.bfloat16, device=dev)
    calls = {"w4a4": lambda: L.bsq_gemm_nvfp4_q(x3q, x3s, gx3, w3q, w3s, g3, y=y3),
             "fp8r": lambda: L.bsq_gemm_fp8r_q(x2q, x2s, w2q, w2s, y=y2)}
    for name, fn in calls.items():
        done = 0.0
        while done < warm_ms:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(8):
                fn()
            e1.record()
            torch.cuda.synchronize()
            done += e0.elapsed_time(e1)
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        print("ran %s: warmed %.0f ms, then %d launches" % (name, done, reps), flush=True)


def _collect(paths, last=5):
    """{kernel key: {counter: mean over the last `last` dispatches}} plus mean durations (ns)."""
    vals, durs = {}, {}
    for path in paths:
        rows = list(csv.DictReader(open(path)))
        per = {}
        for r in rows:
            key = next((k for k in KERNELS if k in r["Kernel_Name"]), None)
            if key is None:
                continue
            d = per.setdefault(key, {}).setdefault(int(r.get("Dispatch_Id", 0)), {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                d["_dur"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
        for key, dispatches in per.items():
            ids = sorted(dispatches)[-last:]
            for cname in {c for i in ids for c in dispatches[i]}:
                xs = [dispatches[i][cname] for i in ids if cname in dispatches[i]]
                if cname == "_dur":
                    durs.setdefault(key, []).extend(xs)
                else:
                    vals.setdefault(key, {})[cname] = sum(xs) / len(xs)
    return vals, {k: sum(v) / len(v) for k, v in durs.items()}


def summarize(*paths):
    vals, durs = _collect(paths)
    print("| quantity | %s |" % " | ".join(KERNELS[k][0] for k in KERNELS if k in vals))
    print("|---|" + "---|" * len([k for k in KERNELS if k in vals]))
    keys = [k for k in KERNELS if k in vals]

    def row(label, f):
        out = []
        for k in keys:
            try:
                out.append(f(vals[k], durs.get(k)))
            except (KeyError, ZeroDivisionError, TypeError):
                out.append("n/a")
        print("| %s | %s |" % (label, " | ".join(out)))

    row("dispatch duration under the profiler (us)", lambda v, d: "%.1f" % (d / 1e3))
    cyc = lambda v: v["GRBM_GUI_ACTIVE"] / XCDS  # clock cycles of the dispatch
    row("cycles = GRBM_GUI_ACTIVE / 8 XCDs", lambda v, d: "%.0f" % cyc(v))
    row("clock = cycles / duration (GHz)", lambda v, d: "%.2f" % (cyc(v) / d))
    row("matrix cores busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs)",
        lambda v, d: "%.3f" % (v["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc(v) * SIMDS)))
    row("VALU issued while the MFMA unit is busy = COEXEC / MFMA_BUSY",
        lambda v, d: "%.3f" % (v["SQ_VALU_MFMA_COEXEC_CYCLES"] / v["SQ_VALU_MFMA_BUSY_CYCLES"]))
    for c in ("SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
              "SQ_ACTIVE_INST_VMEM", "SQ_WAIT_INST_LDS"):
        row("%s / SQ_WAVE_CYCLES" % c, lambda v, d, c=c: "%.3f" % (v[c] / v["SQ_WAVE_CYCLES"]))
    row("SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS",
        lambda v, d: "%.3f" % (v["SQ_LDS_BANK_CONFLICT"] / v["SQ_ACTIVE_INST_LDS"]))
    for c in ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_VMEM"):
        row("%s per dispatch" % c, lambda v, d, c=c: "%.0f" % v[c])
    row("VALU instructions per MFMA", lambda v, d: "%.2f" % (v["SQ_INSTS_VALU"] / v["SQ_INSTS_MFMA"]))
    row("waves resident per SIMD, averaged = SQ_WAVE_CYCLES x 4 / (cycles x 1024)",
        lambda v, d: "%.3f" % (v["SQ_WAVE_CYCLES"] * 4 / (cyc(v) * SIMDS)))
    for k in keys:
        name, flops = KERNELS[k]
        if k in durs:
            print("\n%s: %.1f TFLOP/s under the profiler (%.3f of the %s peak)" % (
                name, flops / durs[k] / 1e3, flops / durs[k] / 1e3 / (2500.0 if "w4a4" in k else 5000.0),
                "f16" if "w4a4" in k else "fp8"))


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        run()
    elif len(sys.argv) >= 3 and sys.argv[1] == "summarize":
        summarize(*sys.argv[2:])
    else:
        raise SystemExit(__doc__)
