"""Markdown summaries of rocprofv3 kernel traces (for the summaries under profiles/).

    python3 -m block_scaled_precision_row_amd.kernel_stats <dir>/run_kernel_stats.csv \\
        [--trace <dir>/run_kernel_trace.csv] [--last N] [--runs MIN] [--match TEXT]

prints the per-kernel table of the stats file (calls, average, minimum and maximum duration in
microseconds, share of the total). With --trace it also groups the dispatches of the trace by
kernel, grid size and workgroup size (one launch shape per row: call count, mean and minimum
duration), and with --last N it gives, per kernel, the mean duration of its last N dispatches
(the steady-state launches of a run that warms up first). With --runs MIN it lists, in launch
order, every run of at least MIN consecutive dispatches of one kernel and grid: its length, median
and minimum duration -- a workload that warms each shape and then times it back to back shows up
as one run per shape. --match TEXT keeps, in every table, only the kernels whose name holds TEXT.
"""
import csv
import sys


def _num(r, *keys):
    for k in keys:
        if k in r and r[k] not in ("", None):
            return float(r[k])
    raise KeyError(keys)


def _short(name, width=90):
    """Kernel name without 'void', anonymous namespaces and the parameter list."""
    name = name.replace("void ", "", 1).replace("(anonymous namespace)::", "")
    depth = 0
    for i, c in enumerate(name):
        depth += c == "<"
        depth -= c == ">"
        if c == "(" and depth == 0 and i > 0:
            name = name[:i]
            break
    return name if len(name) <= width else name[: width - 3] + "..."


def stats_table(path, match=None):
    rows = [r for r in csv.DictReader(open(path)) if not match or match in r["Name"]]
    rows.sort(key=lambda r: -_num(r, "TotalDurationNs"))
    print("| kernel | calls | average us | min us | max us | share of kernel time |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        print("| %s | %d | %.2f | %.2f | %.2f | %.1f %% |" % (
            _short(r["Name"]), int(_num(r, "Calls")), _num(r, "AverageNs") / 1e3, _num(r, "MinNs") / 1e3,
            _num(r, "MaxNs") / 1e3, _num(r, "Percentage")))


def _grid(r):
    try:
        return "%d x %d x %d" % (int(_num(r, "Grid_Size_X", "Grid_Size")), int(_num(r, "Grid_Size_Y")),
                                 int(_num(r, "Grid_Size_Z")))
    except KeyError:
        return str(int(_num(r, "Grid_Size")))


def _wg(r):
    try:
        return "%d" % int(_num(r, "Workgroup_Size_X", "Workgroup_Size"))
    except KeyError:
        return "?"


def trace_tables(path, last=0, match=None):
    rows = [r for r in csv.DictReader(open(path)) if not match or match in r["Kernel_Name"]]
    rows.sort(key=lambda r: _num(r, "Start_Timestamp"))
    shapes = {}
    per_kernel = {}
    for r in rows:
        dur = (_num(r, "End_Timestamp") - _num(r, "Start_Timestamp")) / 1e3
        key = (r["Kernel_Name"], _grid(r), _wg(r))
        shapes.setdefault(key, []).append(dur)
        per_kernel.setdefault(r["Kernel_Name"], []).append(dur)
    print("\n| kernel | grid (threads) | workgroup | calls | mean us | min us |")
    print("|---|---|---|---|---|---|")
    for (name, grid, wg), ds in sorted(shapes.items(), key=lambda kv: -sum(kv[1])):
        print("| %s | %s | %s | %d | %.2f | %.2f |" % (_short(name), grid, wg, len(ds), sum(ds) / len(ds), min(ds)))
    if last:
        print("\n| kernel | mean us of the last %d dispatches |" % last)
        print("|---|---|")
        for name, ds in sorted(per_kernel.items(), key=lambda kv: -sum(kv[1])):
            if len(ds) >= last:
                tail = ds[-last:]
                print("| %s | %.2f |" % (_short(name), sum(tail) / len(tail)))


def run_table(path, min_len, match=None):
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: _num(r, "Start_Timestamp"))
    runs = []
    for r in rows:
        if match and match not in r["Kernel_Name"]:
            key = None
        else:
            key = (r["Kernel_Name"], _grid(r), _wg(r))
        dur = (_num(r, "End_Timestamp") - _num(r, "Start_Timestamp")) / 1e3
        if runs and runs[-1][0] == key:
            runs[-1][1].append(dur)
        else:
            runs.append((key, [dur]))
    print("\n| run | kernel | grid (threads) | workgroup | dispatches | median us | min us |")
    print("|---|---|---|---|---|---|---|")
    n = 0
    for key, ds in runs:
        if key is None or len(ds) < min_len:
            continue
        n += 1
        srt = sorted(ds)
        med = srt[len(srt) // 2] if len(srt) % 2 else 0.5 * (srt[len(srt) // 2 - 1] + srt[len(srt) // 2])
        print("| %d | %s | %s | %s | %d | %.2f | %.2f |" % (n, _short(key[0]), key[1], key[2], len(ds), med, srt[0]))


if __name__ == "__main__":
    args = sys.argv[1:]
    if not args or args[0].startswith("-"):
        raise SystemExit(__doc__)
    trace, last = None, 0
    if "--trace" in args:
        trace = args[args.index("--trace") + 1]
    if "--last" in args:
        last = int(args[args.index("--last") + 1])
    match = args[args.index("--match") + 1] if "--match" in args else None
    stats_table(args[0], match)
    if trace:
        trace_tables(trace, last, match)
    if trace and "--runs" in args:
        run_table(trace, int(args[args.index("--runs") + 1]), match)
