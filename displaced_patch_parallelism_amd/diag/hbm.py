"""Cold- and warm-cache HBM rates of the streaming calls (GroupNorm, band splice) and of a plain copy.

The MI355X keeps a 256 MB Infinity Cache (MALL) in front of HBM, so a call that re-reads the
same band measures the cache, not HBM.  Here every call of a cold run reads and writes a
different buffer set, the sets together exceeding 2 x 256 MB, so each call finds its band in
HBM; the warm run repeats one set.  Each run is captured in one HIP graph and replayed, so the
host's per-call dispatch cost is not timed (a bare launch loop from Python costs about 8 us a
call, more than most of these kernels take).  Rates count one read and one write of the band (the
algorithmic bytes).  Two large copies give the box's practical HBM ceiling: torch's 1 GiB
device copy, and the library's own splice kernel on a 512 MB band (a stream far larger than the
MALL, so the launch's ramp and tail do not count).

    python -m displaced_patch_parallelism_amd.diag.hbm [--configs c1,c4a,c4b] [--reps 3]

prints one JSON line per measurement.
"""

import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

COLD_BYTES = 640 << 20      # buffer sets rotated per cold run: > 2 x the 256 MB MALL


def _time(fn, ks, reps):
    """Best-of-reps GPU time per call (us) of fn(k) for k in ks, replayed from one HIP graph so
    that the host's per-call dispatch cost is not timed."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for k in ks:                       # eager pass: workspace caches settle before capture
            fn(k)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in ks:
            fn(k)
    g.replay()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e3 / len(ks))
    return best


def copy_rate(reps):
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    us = _time(lambda k: dst.copy_(src), range(5), reps)
    return {"op": "copy", "bytes": 2 * n, "us": round(us, 2), "gbs": round(2 * n / us / 1e3, 1)}


def splice_ceiling(reps):
    """The splice kernel on one 512 MB band (1 x 2 x 262144 x 1024 bf16 map, 2 row patches)."""
    import torch
    import displaced_patch_parallelism_amd as dp
    p = dp.Patch(1, 2, 262144, 1024, 2, 1)
    x = torch.empty((1, 1, 262144, 1024), dtype=torch.bfloat16, device="cuda").fill_(1)
    m = torch.empty((1, 2, 262144, 1024), dtype=torch.bfloat16, device="cuda")
    n = x.numel() * 2
    us = _time(lambda k: dp.dp_stale_update(p, x, m), range(5), reps)
    return {"op": "splice_512MB", "bytes": 2 * n, "us": round(us, 2), "gbs": round(2 * n / us / 1e3, 1)}


def call_rates(cfg, reps):
    import torch
    import displaced_patch_parallelism_amd as dp
    from displaced_patch_parallelism_amd.layers import torch_dtype
    dev = torch.device("cuda:0")
    dt = torch_dtype(cfg.dtype)
    p = dp.Patch(cfg.B, cfg.H, cfg.W, cfg.C, cfg.P, cfg.patch)
    band = (cfg.B, cfg.h, cfg.W, cfg.C)
    full = (cfg.B, cfg.H, cfg.W, cfg.C)
    bb = cfg.band_bytes()
    nsets = max(2, -(-COLD_BYTES // (2 * bb)))
    xs = [torch.randn(band, device=dev).to(dt) for _ in range(nsets)]
    ys = [torch.empty(band, dtype=dt, device=dev) for _ in range(nsets)]
    table = torch.randn((cfg.P, cfg.B, cfg.G, 2), device=dev).abs()
    st = torch.empty((cfg.B, cfg.G, 2), device=dev)
    ws = torch.empty(dp.workspace_bytes("groupnorm", p, dp._dtype_code(xs[0]), cfg.G), dtype=torch.uint8, device=dev)
    act = "silu" if "gn_silu" in cfg.graph else None
    gn = lambda k: dp.dp_groupnorm_async(p, xs[k], cfg.G, table, cfg.eps, "corrected", act,
                                         fresh_stats_out=st, y_patch=ys[k], ws=ws)
    # splice: call k copies source band k into band k % P of map k // P, so a cold run also writes
    # a different band every call
    maps = [torch.empty(full, dtype=dt, device=dev) for _ in range(-(-nsets // cfg.P))]
    pk = [dp.Patch(cfg.B, cfg.H, cfg.W, cfg.C, cfg.P, k % cfg.P) for k in range(nsets)]
    sp = lambda k: dp.dp_stale_update(pk[k], xs[k], maps[k // cfg.P])
    out = []
    for name, fn in (("groupnorm", gn), ("splice", sp)):
        warm = _time(lambda k: fn(0), range(20), reps)
        cold = _time(fn, range(nsets), reps)
        out.append({"op": name, "config": cfg.name, "band_bytes": bb, "sets": nsets,
                    "warm_us": round(warm, 2), "warm_gbs": round(2 * bb / warm / 1e3, 1),
                    "cold_us": round(cold, 2), "cold_gbs": round(2 * bb / cold / 1e3, 1)})
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--configs", default="c1,c2,c3,c4a,c4b")
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args()
    import torch
    if not torch.cuda.is_available():
        print("needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    import displaced_patch_parallelism_amd as dp
    from displaced_patch_parallelism_amd.configs import CONFIGS
    dp.lib()
    print(json.dumps(copy_rate(args.reps)), flush=True)
    print(json.dumps(splice_ceiling(args.reps)), flush=True)
    for name in args.configs.split(","):
        for row in call_rates(CONFIGS[name], args.reps):
            print(json.dumps(row), flush=True)


if __name__ == "__main__":
    main()
