"""The nvfp4 W4A4 GEMM 4096x12288x3072 on operands that toggle few bits against the benchmark's.

The same launch (same shapes, same instructions) is timed on two operand sets:
  low   : positive E2M1 codes (random magnitudes), every block scale 1.0, global scales 1;
  bench : the benchmark's synthetic bf16 activations and weights quantized by the library's
          own quantizers with calibrated global scales (what bench.py times).
A difference in time at equal instruction counts comes from the clock, which the power limit
lowers when more bits switch. Run on one MI355X:

  python3 -m block_scaled_precision_row_amd.operand_bits run
      prints each set's mean launch time (HIP events, after about 100 ms of warm-up);
  cd /tmp && export TMPDIR=/tmp PYTHONPATH=<repo>
  rocprofv3 --pmc GRBM_GUI_ACTIVE -d <d> -o run --output-format csv -- \\
      python3 -m block_scaled_precision_row_amd.operand_bits run
  python3 -m block_scaled_precision_row_amd.operand_bits summarize <d>/run_counter_collection.csv
      prints each set's clock (GRBM_GUI_ACTIVE / 8 XCDs per dispatch, over its duration) from the
      timed launches of the profiled run.
"""
import csv
import sys

M, N, K = 4096, 12288, 3072
WARM, TIMED = 450, 50   # launches per set: warm-up (about 100 ms), then timed


def run():
    import torch

    from block_scaled_precision_row_amd import _lib as L
    from block_scaled_precision_row_amd import synthetic as syn

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    sets = {}
    # low: positive magnitudes in both nibbles, block scales 1.0 (E4M3 0x38), global scales 1.0
    wq = (torch.randint(0, 256, (N, K // 2), generator=gen, device=dev, dtype=torch.int32) & 0x77).to(torch.uint8)
    xq = (torch.randint(0, 256, (M, K // 2), generator=gen, device=dev, dtype=torch.int32) & 0x77).to(torch.uint8)
    one = torch.ones(1, dtype=torch.float32, device=dev)
    sets["low"] = (xq, torch.full((M, K // 16), 0x38, dtype=torch.uint8, device=dev), one, wq,
                   torch.full((N, K // 16), 0x38, dtype=torch.uint8, device=dev), one)
    up = lambda bits: torch.from_numpy(bits.view("int16")).to(dev).view(torch.bfloat16)
    x = up(syn.activations(syn.NVFP4_UP, M, K))
    w = up(syn.weights(syn.NVFP4_UP, N, K))
    gx, gw = L.bsq_calibrate_global_scale(x), L.bsq_calibrate_global_scale(w)
    sets["bench"] = (*L.bsq_quantize_act_nvfp4(x, gx), gx, *L.bsq_quantize_act_nvfp4(w, gw), gw)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    for name, ops in sets.items():
        for _ in range(WARM):
            L.bsq_gemm_nvfp4_q(*ops, y=y)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(TIMED):
            L.bsq_gemm_nvfp4_q(*ops, y=y)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / TIMED * 1e3
        print("%-5s operands: %.1f us per launch, %.1f TFLOP/s, %.3f of the 2.5 PF/s f16 peak"
              % (name, us, 2.0 * M * N * K / (us * 1e-6) / 1e12, 2.0 * M * N * K / (us * 1e-6) / 2.5e15), flush=True)


def summarize(path):
    disp = {}  # dispatch id -> [GRBM_GUI_ACTIVE summed over its rows, duration in ns]
    for r in csv.DictReader(open(path)):
        if "gemm_w4a4_kernel" not in r["Kernel_Name"] or r["Counter_Name"] != "GRBM_GUI_ACTIVE":
            continue
        d = disp.setdefault(int(r["Dispatch_Id"]), [0.0, 0.0])
        d[0] += float(r["Counter_Value"])
        d[1] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    rows = [disp[k] for k in sorted(disp)]
    per = WARM + TIMED
    if len(rows) < 2 * per:
        raise SystemExit("expected %d W4A4 dispatches, found %d" % (2 * per, len(rows)))
    rows = rows[-2 * per:]
    print("| operands | mean dispatch (us) | cycles (GRBM_GUI_ACTIVE / 8) | clock (GHz) | fraction of the f16 peak |")
    print("|---|---|---|---|---|")
    for i, name in enumerate(("low", "bench")):
        timed = rows[i * per + WARM:(i + 1) * per]
        dur = sum(r[1] for r in timed) / len(timed) / 1e3  # us
        cyc = sum(r[0] for r in timed) / len(timed) / 8
        print("| %s | %.1f | %.0f | %.2f | %.3f |" % (name, dur, cyc, cyc / (dur * 1e3),
                                                     2.0 * M * N * K / (dur * 1e-6) / 2.5e15))


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        run()
    elif len(sys.argv) == 3 and sys.argv[1] == "summarize":
        summarize(sys.argv[2])
    else:
        raise SystemExit(__doc__)
