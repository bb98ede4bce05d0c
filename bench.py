#!/usr/bin/env python
"""Benchmark of one displaced-patch step on one MI355X.

A step is patch i's share of one denoising step of the workload's layers, every call of the
hot path in order: corrected asynchronous GroupNorm (statistics, combine, normalise + SiLU),
the 3x3 conv with stale halo rows and/or the attention over spliced K/V; each call writes its
output straight into the resident stale state the next step reads (the fresh band of every
consumer's map and the fresh GroupNorm moments), so no separate splice is needed.  The
default workload is the 3840px pair of layers (c4): the 480x480x320 conv layer (GN+SiLU,
conv3x3 320->320) and the 240x240x640 attention layer (GN, 10x64 attention, 7200 queries
over 57600 stale-spliced keys), 8 row patches, patch 1, one step running both.  Inputs are
seeded synthetic tensors already resident in HBM; each layer's stale state comes from a
synchronous warm-up step run by the same library.

Prints one JSON line: whole-step TFLOP/s (algorithmic conv + attention (+ learned
projection) flops over the wall time of K steps run as replays of a HIP graph that holds
several consecutive steps, between two device synchronisations; the eager, host-launched
step time is reported beside it), per-layer step times, per-call times (a graph of
back-to-back launches of each call, timed with HIP events on the stream it runs on), the
GroupNorm and splice HBM rates cold (buffer sets rotated past the 256 MB MALL) and warm, the
roofline of the dominant kernel, and the CPU oracle's rate on a bounded sample of the same
step.
"""

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "displaced-patch layer TFLOP/s (% bf16 MFMA peak) + GroupNorm/splice HBM GB/s"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense MFMA bf16; fp32 vector
PEAK_HBM_GBS = 8000.0

# source file of each call's main kernel (for the counter file's staleness check)
KERNEL_SOURCES = {"conv": "k_conv.hip", "conv_res": "k_conv.hip", "attn": "k_attention.hip",
                  "gn": "k_groupnorm.hip", "gn_silu": "k_groupnorm.hip", "stale_update": "k_splice.hip",
                  "proj_qkv": "k_linear.hip", "proj_o": "k_linear.hip"}
for _g in ("gn", "gn_silu"):
    for _c in ("conv", "conv_res"):
        KERNEL_SOURCES[f"{_g}+{_c}"] = "k_conv.hip"     # GroupNorm folded into the conv
PROJ_CALLS = ("proj_qkv", "proj_o")


def step_flops(cfg):
    """Algorithmic flops of one patch step: conv + attention + learned projections."""
    return cfg.conv_flops() + cfg.attn_flops() + cfg.proj_flops()


def call_flops(cfg, name):
    """Algorithmic flops of one call of the step (one conv, one attention, one projection)."""
    if name.split("+")[-1] in ("conv", "conv_res"):
        return cfg.conv_flops() / max(cfg.n_conv, 1)
    if name == "attn":
        return cfg.attn_flops() / max(cfg.n_attn, 1)
    if name in PROJ_CALLS:          # the Q/K/V launch is three of the step's four projections
        return cfg.proj_flops() / max(4 * cfg.n_proj, 1) * (3 if name == "proj_qkv" else 1)
    return 0


def kernel_name(op, cfg, cout=None):
    """Main kernel of a call: the bf16 conv picks its tile kernel from the map size (the
    library's plan: 128x160 tiles when at least 384 of them exist, else 64x80 tiles; with a
    GroupNorm folded in, 256x160 tiles where they need no more rounds than the 128x160 ones)."""
    if op == "attn":
        return "attn_bf16_d64_kernel" if cfg.dtype == "bf16" else "attn_f32_kernel"
    if op in PROJ_CALLS:
        return "linear_bf16_kernel" if cfg.dtype == "bf16" else "linear_f32_kernel"
    if op.split("+")[-1] in ("conv", "conv_res"):
        if cfg.dtype != "bf16":
            return "conv3x3_f32_direct_kernel"
        cout = cout or cfg.C
        big = cfg.B * -(-cfg.h // 4) * -(-cfg.W // 32) * -(-cout // 160)
        big8 = cfg.B * -(-cfg.h // 8) * -(-cfg.W // 32) * -(-cout // 160)
        if "+" in op and big >= 384 and -(-big8 // 256) <= -(-big // 512):
            # with a GroupNorm folded in (its lanes and parameter table fit the kernel's LDS)
            return "conv3x3_bf16_gn_tile8_kernel"
        return "conv3x3_bf16_halo_tile_kernel" if big >= 384 else "conv3x3_bf16_halo_wave8_kernel"
    return op


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(name):
    path = os.path.join(ROOT, "displaced_patch_parallelism_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if taken on the current source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    ent = table.get(f"{kernel}/{workload}")
    if not ent or ent.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return ent.get("hbm_bytes_per_launch")


def host_description():
    """The host the CPU baseline ran on: logical CPUs, model name, thread settings."""
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"os_cpu_count": os.cpu_count(), "affinity_cpus": affinity, "cpu_model": model,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def oracle_patch_step(cfg, params, xb, state, i, rows):
    """The oracle's displaced step of patch i; an attention that ends the graph is computed on
    the query rows ``rows`` only (None: all).  Returns the algorithmic flops computed."""
    import numpy as np
    import oracle
    if rows is None or not cfg.graph[-1] == "attn":
        oracle.displaced_layer(cfg.graph, params, xb, state, cfg.P, i)
        return step_flops(cfg)
    head = cfg.graph[:-1]
    step_of = lambda key: key[0] if isinstance(key, tuple) else key  # noqa: E731
    sub_state = {"stats": {k: t for k, t in state["stats"].items() if k < len(head)},
                 "maps": {k: m for k, m in state["maps"].items() if step_of(k) < len(head)}}
    h = xb
    if head:
        outs, _ = oracle.displaced_layer(head, params, xb, sub_state, cfg.P, i)
        h = outs[-1]
    B, hb, W, C = h.shape
    k = len(cfg.graph) - 1
    tok = np.asarray(h, dtype=np.float64).reshape(B, hb * W, C)
    st = np.asarray(state["maps"][k], dtype=np.float64).reshape(B, cfg.N, C)
    oracle.attention_splice(tok, tok, tok, st, st, cfg.H, cfg.W, cfg.P, i, cfg.heads, rows=rows)
    return step_flops(cfg) - cfg.attn_flops() + cfg.attn_flops() * len(rows) / cfg.Nq


def cpu_baseline(parts, seconds, seed):
    """The oracle's displaced step of the same patches, repeated for about `seconds`; an
    attention whose full oracle would take minutes (more than 1e11 flops) runs on a seeded
    sample of 256 query rows."""
    import numpy as np
    import oracle
    prepared = []
    for cfg, inp, i in parts:
        params = {"G": cfg.G, "eps": cfg.eps, "heads": cfg.heads, "convs": inp.convs, "projs": inp.projs}
        _, state = oracle.sync_layer(cfg.graph, params, inp.x_prev, cfg.P, state_only=True)
        xb = inp.x[:, i * cfg.h:(i + 1) * cfg.h]
        rows = None
        if cfg.attn_flops() > 1e11 and cfg.graph[-1] == "attn":
            rows = np.sort(np.random.default_rng(seed).choice(cfg.Nq, 256, replace=False))
        prepared.append((cfg, params, xb, state, i, rows))
    reps, flops = 0, 0.0
    t0 = time.perf_counter()
    while True:
        for cfg, params, xb, state, i, rows in prepared:
            flops += oracle_patch_step(cfg, params, xb, state, i, rows)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    desc = []
    for cfg, _, _, _, i, rows in prepared:
        what = "+".join(cfg.graph)
        if rows is not None:
            what += f", attention on {len(rows)} of {cfg.Nq} query rows"
        desc.append(f"{cfg.name} patch {i} ({what})")
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{reps} x oracle displaced step of " + "; ".join(desc) + f" (float64 numpy) in {el:.1f} s",
            "seconds_per_step": el / reps, "host": host_description()}


def capture_steps(layers, steps):
    """``steps`` consecutive steps of every (layer, x_patch, i), in order, as one HIP graph."""
    import torch
    dev = layers[0][0].device
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for _ in range(2):
            for layer, xb, i in layers:
                layer.step(xb, i)
    torch.cuda.current_stream(dev).wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            for layer, xb, i in layers:
                layer.step(xb, i)
    return graph


def time_graph(graph, replays):
    import torch
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(replays):
        graph.replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c4",
                    help="workload: c4 (default: c4a + c4b), or one layer: c0, c1, c2, c3, c4a, c4b, c2p, c4bp, "
                         "c1r, c2t")
    ap.add_argument("--patch", type=int, default=None, help="patch index (default: the config's)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle sample length; 0 skips it")
    ap.add_argument("--no-hbm", action="store_true", help="skip the cold/warm GroupNorm and splice rates")
    ap.add_argument("--seed", type=int, default=0)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one patch's step on ONE GPU; the exchange between GPUs is not "
              "implemented, so --gpus must be 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import displaced_patch_parallelism_amd as dp
    from displaced_patch_parallelism_amd import synth
    from displaced_patch_parallelism_amd.configs import COMPOSITES, CONFIGS
    from displaced_patch_parallelism_amd.diag import hbm
    from displaced_patch_parallelism_amd.layers import DisplacedLayer

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    dp.lib()  # fail loudly if the library is not built
    names = COMPOSITES.get(args.config, (args.config,))
    cfgs = [CONFIGS[n] for n in names]
    composite = len(cfgs) > 1
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} ({getattr(props, 'gcnArchName', '?')}), {props.multi_processor_count} CUs; "
        f"workload {args.config}: " + "; ".join(f"{c.name}: {c.note}" for c in cfgs))

    parts = []       # (cfg, inp, layer, x_patch, i)
    for cfg in cfgs:
        i = cfg.patch if args.patch is None else args.patch
        inp = synth.layer_inputs(cfg, args.seed)
        layer = DisplacedLayer(cfg, inp.convs, dev, projs=inp.projs)
        to = lambda a, layer=layer: torch.from_numpy(a).to(dev, layer.dt).contiguous()  # noqa: E731
        layer.warmup(to(inp.x_prev))             # previous step: synchronous, builds the stale state
        x_patch = to(inp.x[:, i * cfg.h:(i + 1) * cfg.h])
        parts.append((cfg, inp, layer, x_patch, i))
        log(f"{cfg.name}: warm-up done, patch {i}")
    torch.cuda.synchronize()
    steps = [(layer, xb, i) for _, _, layer, xb, i in parts]

    for _ in range(args.warmup):
        for layer, xb, i in steps:
            layer.step(xb, i)
    torch.cuda.synchronize()

    # eager steps (host launches every call), for reference
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for layer, xb, i in steps:
            layer.step(xb, i)
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t0

    # U consecutive steps captured once as a HIP graph; the K timed steps are K/U replays
    unroll = next(u for u in (10, 8, 5, 4, 2, 1) if args.steps % u == 0)
    graph = capture_steps(steps, unroll)
    for _ in range(max(1, args.warmup // unroll)):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps // unroll):
        graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del graph
    log(f"timed {args.steps} steps: {1e3 * wall / args.steps:.4f} ms per step")

    # each layer's own step time (a graph of its steps alone), for a composite workload
    layer_ms = {}
    if composite:
        for (cfg, _, layer, xb, i) in parts:
            g = capture_steps([(layer, xb, i)], 2)
            reps = 3 if step_flops(cfg) > 1e11 else 20
            layer_ms[cfg.name] = 1e3 * time_graph(g, reps) / (2 * reps)
            del g

    # per call: a graph of R back-to-back launches of that call, timed with HIP events on the
    # stream it runs on (the current stream, where the library launches)
    per_call_us = {}
    for (cfg, _, layer, xb, i) in parts:
        for name, fn, _ in layer.calls(xb, i):
            reps = 2 if call_flops(cfg, name) > 1e11 else 20
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(reps):
                    fn()
            g.replay()
            torch.cuda.synchronize()
            stream = torch.cuda.current_stream(dev)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(5):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            key = f"{cfg.name}/{name}" if composite else name
            per_call_us[key] = (cfg, name, 1e3 * e0.elapsed_time(e1) / (5 * reps))
            del g
    log("per-call times done")

    ms_per_step = 1e3 * wall / args.steps
    flops = sum(step_flops(c) for c in cfgs)
    value = flops / (ms_per_step * 1e-3) / 1e12
    dtype = cfgs[0].dtype
    peak = PEAK_TFLOPS[dtype]

    kernels = {}
    for key, (cfg, name, us) in per_call_us.items():
        ent = {"us": round(us, 3)}
        if call_flops(cfg, name):
            ent["tflops"] = round(call_flops(cfg, name) / (us * 1e-6) / 1e12, 2)
            ent["frac_mfma_peak"] = round(ent["tflops"] / peak, 4)
        elif name in ("gn", "gn_silu", "stale_update"):
            gbs = 2 * cfg.band_bytes() / (us * 1e-6) / 1e9       # one read + one write of the band
            ent["gbs_warm"] = round(gbs, 1)
            ent["frac_hbm_peak_warm"] = round(gbs / PEAK_HBM_GBS, 4)
        kernels[key] = ent

    # GroupNorm and splice, cold (every call on its own buffers, > 2x the MALL) and warm
    hbm_rates = {}
    if not args.no_hbm:
        hbm_rates["copy"] = hbm.copy_rate(3)
        hbm_rates["splice_512MB"] = hbm.splice_ceiling(3)
        for cfg in cfgs:
            for row in hbm.call_rates(cfg, 3):
                ent = {k: row[k] for k in ("band_bytes", "sets", "warm_us", "warm_gbs", "cold_us", "cold_gbs")}
                ent["frac_hbm_peak_cold"] = round(row["cold_gbs"] / PEAK_HBM_GBS, 4)
                ent["frac_copy_cold"] = round(row["cold_gbs"] / hbm_rates["copy"]["gbs"], 4)
                ent["frac_splice_512MB_cold"] = round(row["cold_gbs"] / hbm_rates["splice_512MB"]["gbs"], 4)
                hbm_rates[f"{cfg.name}/{row['op']}"] = ent
        log("HBM rates done")

    compute = [k for k, (cfg, name, _) in per_call_us.items() if call_flops(cfg, name)]
    dom = max(compute, key=lambda k: per_call_us[k][2])
    dcfg, dname, dus = per_call_us[dom]
    dom_flops = call_flops(dcfg, dname)
    achieved = dom_flops / (dus * 1e-6) / 1e12
    roofline = {"bound": "mfma", "kernel": kernel_name(dname, dcfg), "call": dom, "achieved": round(achieved, 2),
                "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": traffic_for(dname, dcfg.name), "algorithmic_flops_per_launch": dom_flops,
                "launch_us": round(dus, 3)}

    if composite:
        workload = f"{args.config}: " + " + ".join(f"{c.name} ({c.note})" for c in cfgs)
    else:
        workload = f"{cfgs[0].name}: {cfgs[0].note}"
    config = {"workload": workload,
              "layers": [{"name": c.name, "map": [c.B, c.H, c.W, c.C], "groups": c.G, "patches": c.P,
                          "patch": i, "graph": list(c.graph),
                          **({"heads": c.heads, "head_dim": c.head_dim} if c.has_attn else {})}
                         for c, _, _, _, i in parts],
              "parallelism": "one patch on one GPU"}
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_eager": round(1e3 * wall_eager / args.steps, 5),
        "steps_per_graph": unroll,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,1) activations, previous step x+0.05*N(0,1), N(0,1/fan_in) weights)",
        "config": config,
        "step_gflop": round(flops / 1e9, 3),
        "frac_mfma_peak": round(value / peak, 4),
    }
    if layer_ms:
        line["layers_ms_per_step"] = {k: round(v, 5) for k, v in layer_ms.items()}
    line["kernels"] = kernels
    if hbm_rates:
        line["hbm"] = hbm_rates
    line["roofline"] = roofline
    if args.cpu_seconds > 0:
        log("timing the CPU oracle ...")
        line["cpu_baseline"] = cpu_baseline([(c, inp, i) for c, inp, _, _, i in parts], args.cpu_seconds,
                                            args.seed)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
