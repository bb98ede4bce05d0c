"""Several denoising steps of one layer, every patch displaced, against the synchronous layer.

Runs on one GPU what a P-device DistriFusion run does to one layer: a
synchronous warm-up step on x_0, then for t = 1..T every patch's displaced step
on x_t against the state of step t-1, the gathered fresh bands and moments
becoming the state of step t (study.space page, Method; DistriFusion summary on
atlas.scime.ai, Approach and the warm-up rows of "Measured effects reported in
the paper").  Each GroupNorm mode (corrected; local statistics only; stale
statistics only) runs as its own layer instance on the same trajectory, and at
every step its final output is compared with the synchronous layer's output
on x_t (exact statistics, no stale context).

The trajectory is synthetic: x_0 ~ N(0, 1), x_t = x_{t-1} + 0.05 N(0, 1)
(``synth.trajectory``).

    python -m displaced_patch_parallelism_amd.trajectory --config c1 --steps 6

prints one JSON line per step with the relative L2 distance of each mode's
output from the synchronous output, and the time of an all-patch step.
"""

import argparse
import json
import sys

import torch

from . import lib, synth
from .configs import CONFIGS
from .layers import DisplacedLayer

MODES = ("corrected", "local", "stale")


def rel_l2(a, b):
    a, b = a.float(), b.float()
    return float((a - b).norm() / b.norm())


def run(cfg, steps, seed=0, modes=MODES, device="cuda:0", log=None):
    """Yields, per step t = 1..steps, {mode: relative L2 drift of the final output}."""
    dev = torch.device(device)
    tr = synth.trajectory(cfg, seed, steps)
    sync = DisplacedLayer(cfg, tr.convs, dev, projs=tr.projs)
    layers = {m: DisplacedLayer(cfg, tr.convs, dev, projs=tr.projs) for m in modes}
    to = lambda a: torch.from_numpy(a).to(dev, sync.dt).contiguous()  # noqa: E731
    x0 = to(tr.xs[0])
    for layer in layers.values():
        layer.warmup(x0)
    for t in range(1, steps + 1):
        xt = to(tr.xs[t])
        ref = sync.warmup(xt)[-1]
        row = {"step": t}
        for m, layer in layers.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            out = layer.step_all(xt, gn_mode=m)[-1]
            e1.record()
            torch.cuda.synchronize()
            row[m] = rel_l2(out, ref)
            row[f"{m}_ms"] = round(e0.elapsed_time(e1), 4)
        if log:
            log(row)
        yield row


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--config", default="c1")
    ap.add_argument("--steps", type=int, default=6)
    ap.add_argument("--seed", type=int, default=0)
    args = ap.parse_args()
    if not torch.cuda.is_available():
        print("needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    lib()
    cfg = CONFIGS[args.config]
    for row in run(cfg, args.steps, args.seed):
        row["config"] = cfg.name
        print(json.dumps(row), flush=True)


if __name__ == "__main__":
    main()
