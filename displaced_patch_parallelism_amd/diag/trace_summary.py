"""Per-kernel duration statistics of a rocprofv3 kernel trace, as a markdown table.

    python -m displaced_patch_parallelism_amd.diag.trace_summary TRACE [--skip N]

TRACE is the *_kernel_trace.csv that `rocprofv3 --kernel-trace --output-format csv -d DIR
-o NAME` wrote (DIR/NAME_kernel_trace.csv), or DIR itself (the trace files directly in it).
For every kernel: dispatches, median, mean, min and max duration (End_Timestamp -
Start_Timestamp, ns -> us), and its share of the summed time.  --skip N leaves out each
kernel's first N dispatches (warm-up calls).
"""

import argparse
import collections
import csv
import glob
import os
import statistics
import sys


def kernel_durations(trace):
    """{kernel name: [duration us, in dispatch order]} from a run's kernel trace."""
    paths = [trace] if os.path.isfile(trace) else glob.glob(os.path.join(trace, "*kernel_trace.csv"))
    if not paths:
        raise SystemExit(f"no *kernel_trace.csv in {trace}")
    rows = []
    for path in paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                rows.append((int(r["Start_Timestamp"]), r["Kernel_Name"],
                             (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    rows.sort()
    out = collections.defaultdict(list)
    for _, name, us in rows:
        out[name].append(us)
    return out


def short_name(name):
    name = name.replace("dp::(anonymous namespace)::", "").split("(")[0]
    return name[5:] if name.startswith("void ") else name


def table(trace, skip=0):
    durs = {k: v[skip:] for k, v in kernel_durations(trace).items() if len(v) > skip}
    total = sum(sum(v) for v in durs.values())
    lines = ["| kernel | dispatches | median us | mean us | min us | max us | % time |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{short_name(name)}` | {len(v)} | {statistics.median(v):.3f} | {statistics.fmean(v):.3f} | "
                     f"{min(v):.3f} | {max(v):.3f} | {100.0 * sum(v) / total:.1f} |")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("trace")
    ap.add_argument("--skip", type=int, default=0)
    args = ap.parse_args()
    print(table(args.trace, args.skip))


if __name__ == "__main__":
    sys.exit(main())
