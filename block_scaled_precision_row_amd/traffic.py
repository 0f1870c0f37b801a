"""Measure the HBM traffic of the W4A4 GEMM at the benchmark shape with rocprofv3 counters.

Two steps, run on one MI355X:

  1. the workload, once under each counter (FETCH_SIZE, then WRITE_SIZE), from any directory
     with the repository on the module path (cd /tmp && export TMPDIR=/tmp PYTHONPATH=<repo>):
         rocprofv3 --pmc FETCH_SIZE -d <d1> -o run --output-format csv -- python3 -m block_scaled_precision_row_amd.traffic run
         rocprofv3 --pmc WRITE_SIZE -d <d2> -o run --output-format csv -- python3 -m block_scaled_precision_row_amd.traffic run
     It launches a plain device copy of a known size (torch's copy kernel,
     COPY_BYTES read and COPY_BYTES written) and then the nvfp4 W4A4 GEMM
     4096x12288x3072 a few times.
  2. python3 -m block_scaled_precision_row_amd.traffic summarize <d1>/run_counter_collection.csv \\
         <d2>/run_counter_collection.csv
     scales each counter by COPY_BYTES / (the counter's reading for the copy kernel),
     takes the GEMM's mean per launch and writes
     profiles/gemm_w4a4_4096x12288x3072_traffic.json with the hash of the kernel's sources.
"""
import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
# the W4A4 kernel and every header it includes: a change to any of them makes a stored count stale
SOURCES = [os.path.join(CSRC, f) for f in ("gemm_w4a4.hip", "gemm_common.hpp", "gemm_tiles.hpp", "bsq_device.hpp",
                                            "bsq_launch.hpp")]


def source_hash():
    h = hashlib.sha256()
    for path in SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()
OUT = os.path.join(ROOT, "profiles", "gemm_w4a4_4096x12288x3072_traffic.json")
COPY_BYTES = 256 << 20
M, K, N = 4096, 3072, 12288


def run(reps=3):
    import torch

    from block_scaled_precision_row_amd import _lib as L
    from block_scaled_precision_row_amd import synthetic as syn

    dev = torch.device("cuda:0")
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    up = lambda bits: torch.from_numpy(bits.view("int16")).to(dev).view(torch.bfloat16)
    x = up(syn.activations(syn.NVFP4_UP, M, K))
    w = up(syn.weights(syn.NVFP4_UP, N, K))
    g = L.bsq_calibrate_global_scale(w)
    wq, ws = L.bsq_quantize_act_nvfp4(w, g)
    gx = L.bsq_calibrate_global_scale(x)
    xq, xs = L.bsq_quantize_act_nvfp4(x, gx)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    for _ in range(reps):
        L.bsq_gemm_nvfp4_q(xq, xs, gx, wq, ws, g, y=y)
    torch.cuda.synchronize()
    print("ran copy x2 and gemm_w4a4 x%d" % reps)


def _per_kernel(path, counter):
    vals = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)  # KiB -> bytes
    return vals


def summarize(fetch_csv, write_csv):
    out = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = _per_kernel(path, name)
        copy = [v for k, vs in vals.items() if "copy" in k.lower() or "elementwise" in k.lower() for v in vs]
        gemm = [v for k, vs in vals.items() if "gemm_w4a4" in k for v in vs]
        if not copy or not gemm:
            raise SystemExit("counter %s: copy or GEMM dispatches not found in %s" % (name, path))
        factor = COPY_BYTES / (sum(copy) / len(copy))
        out[name] = {"copy_reading_bytes": sum(copy) / len(copy), "factor": factor,
                     "gemm_reading_bytes": sum(gemm) / len(gemm), "gemm_bytes": factor * sum(gemm) / len(gemm)}
    total = out["FETCH_SIZE"]["gemm_bytes"] + out["WRITE_SIZE"]["gemm_bytes"]
    algorithmic = M * K // 2 + M * K // 16 + N * K // 2 + N * K // 16 + M * N * 2
    sha = source_hash()
    res = {"kernel": "gemm_w4a4_kernel<256, 256, false, 1> (no adapter)", "shape": "4096x12288x3072", "bytes_per_launch": round(total),
           "algorithmic_bytes_per_launch": algorithmic, "counters": out, "source_sha256": sha,
           "copy_bytes": COPY_BYTES}
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    with open(OUT, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        run()
    elif len(sys.argv) == 4 and sys.argv[1] == "summarize":
        summarize(sys.argv[2], sys.argv[3])
    else:
        raise SystemExit(__doc__)
