"""HBM traffic of one kernel from rocprofv3 counters, calibrated on a plain copy.

FETCH_SIZE and WRITE_SIZE (KiB per dispatch, L2 <-> memory) are collected in
two separate `rocprofv3 --pmc` runs, each of which fits the TCC counter budget.
The same two counters are read for a plain device-to-device copy of a known
size; the ratio known bytes / counted bytes scales the kernel's counts.

  python -m displaced_patch_parallelism_amd.diag.traffic copy [MiB]
      the calibration workload: torch copies of MiB MiB (default 64), 10 times
  python -m displaced_patch_parallelism_amd.diag.traffic summarize KERNEL \
        FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR [MiB]
      prints one JSON object: per-dispatch means and the calibrated bytes
"""

import collections
import csv
import glob
import json
import os
import sys


def per_dispatch(run_dir, name_part, counter):
    """Mean over dispatches of `counter` for kernels whose name contains name_part."""
    vals = collections.defaultdict(float)
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if name_part in row["Kernel_Name"] and row["Counter_Name"] == counter:
                    vals[row["Dispatch_Id"]] += float(row["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for {name_part!r} under {run_dir}")
    return sum(vals.values()) / len(vals), len(vals)


def copy(mib=64, reps=10):
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB x {reps}", flush=True)


def summarize(kernel, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, mib=64):
    fk, nf = per_dispatch(fetch_dir, kernel, "FETCH_SIZE")
    wk, nw = per_dispatch(write_dir, kernel, "WRITE_SIZE")
    # a device-to-device tensor copy runs as the HIP runtime's copyBuffer blit kernel
    cf, _ = per_dispatch(copy_fetch_dir, "copyBuffer", "FETCH_SIZE")
    cw, _ = per_dispatch(copy_write_dir, "copyBuffer", "WRITE_SIZE")
    known_kib = mib * 1024
    f_scale, w_scale = known_kib / cf, known_kib / cw
    out = {
        "kernel": kernel,
        "fetch_kib_per_dispatch": round(fk, 1), "fetch_dispatches": nf,
        "write_kib_per_dispatch": round(wk, 1), "write_dispatches": nw,
        "copy_mib": mib, "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1),
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
        "hbm_bytes_per_launch": int(round((fk * f_scale + wk * w_scale) * 1024)),
    }
    print(json.dumps(out))
    return out


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "copy":
        copy(int(sys.argv[2]) if len(sys.argv) > 2 else 64)
    elif len(sys.argv) >= 7 and sys.argv[1] == "summarize":
        summarize(*sys.argv[2:7], *([int(sys.argv[7])] if len(sys.argv) > 7 else []))
    else:
        print(__doc__)
        sys.exit(2)
