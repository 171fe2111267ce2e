#!/usr/bin/env python3
"""Markdown summary of a rocprofv3 ``--kernel-trace --stats`` run.

    rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- python3 bench.py --workload 1.6b-32k
    python3 -m hbm_bandwidth_bound_amd.stats_profile --dir <dir> --title "bench.py at 1.6b-32k" \\
        --command "<the rocprofv3 command>" --out profiles/<kernel>_<workload>_stats.md

Reads every ``*kernel_stats.csv`` under ``--dir`` (rocprofv3's per-kernel totals: calls, total,
average, minimum and maximum duration) and writes one table, the decoder's kernels first, with
each kernel's share of the GPU time. Kernels whose names do not start with ``kie::`` (torch's
set-up work: weight generation, copies) are folded into one line.
"""
import argparse
import csv
import glob
import os


def read_stats(d):
    rows = {}
    for f in glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r.get("Name") or r.get("KernelName") or r.get("Kernel_Name")
                if not name:
                    continue
                calls = int(float(r.get("Calls", 0)))
                total = float(r.get("TotalDurationNs", 0))
                mn = float(r.get("MinNs", 0))
                mx = float(r.get("MaxNs", 0))
                a = rows.setdefault(name, [0, 0.0, float("inf"), 0.0])
                a[0] += calls
                a[1] += total
                a[2] = min(a[2], mn)
                a[3] = max(a[3], mx)
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--dir", required=True)
    ap.add_argument("--title", required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--note", default="")
    ap.add_argument("--out", required=True)
    args = ap.parse_args()
    rows = read_stats(args.dir)
    if not rows:
        raise SystemExit(f"no kernel_stats.csv under {args.dir}")
    grand = sum(v[1] for v in rows.values())
    ours = sorted(((k, v) for k, v in rows.items() if "kie::" in k), key=lambda kv: -kv[1][1])
    other = [v for k, v in rows.items() if "kie::" not in k]
    L = [f"# rocprofv3 kernel statistics: {args.title}", "", "Command (repository root, MI355X):", "",
         f"    {args.command}", ""]
    if args.note:
        L += [args.note, ""]
    L += ["| kernel | calls | average ms | min ms | max ms | share of GPU time |", "|---|---|---|---|---|---|"]
    for k, (calls, total, mn, mx) in ours:
        L.append(f"| `{k}` | {calls} | {total / max(calls, 1) / 1e6:.4f} | {mn / 1e6:.4f} | {mx / 1e6:.4f} | "
                 f"{100 * total / grand:.2f}% |")
    if other:
        t = sum(v[1] for v in other)
        L.append(f"| (torch set-up kernels: weight generation, copies; {len(other)} kinds) | "
                 f"{sum(v[0] for v in other)} | | | | {100 * t / grand:.2f}% |")
    with open(args.out, "w") as f:
        f.write("\n".join(L) + "\n")
    print("\n".join(L))


if __name__ == "__main__":
    main()
