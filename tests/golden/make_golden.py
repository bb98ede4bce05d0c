"""Writes tests/golden/tiny_layer.json from the oracle alone.

Run from the repository root:  python tests/golden/make_golden.py
The fixture is a regression lock on the oracle: a tiny map (4x4, C=4, G=2,
P=2, one attention head) through GN+SiLU -> conv3x3 with stale halo ->
attention over spliced K/V, patch 1, with the previous step's state made by
the oracle's synchronous layer on x' = x + 0.05 eps (seed 0).
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from displaced_patch_parallelism_amd import synth  # noqa: E402
from displaced_patch_parallelism_amd.configs import LayerConfig  # noqa: E402

CFG = LayerConfig("tiny", "f32", B=1, H=4, W=4, C=4, G=2, P=2,
                  graph=("gn_silu", "conv", "attn"), heads=1, head_dim=4)


def build():
    inp = synth.layer_inputs(CFG, seed=0)
    params = {"G": CFG.G, "eps": CFG.eps, "heads": CFG.heads, "convs": inp.convs}
    _, prev = oracle.sync_layer(CFG.graph, params, inp.x_prev, CFG.P)
    outs, _ = oracle.displaced_layer(CFG.graph, params, inp.x[:, 2:4], prev, CFG.P, 1)
    return {
        "description": "oracle outputs of the tiny displaced layer, patch 1 of 2, seed 0",
        "graph": list(CFG.graph),
        "outputs": [[float(v) for v in o.ravel()] for o in outs],
    }


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_layer.json")
    with open(path, "w") as f:
        json.dump(build(), f, indent=1)
    print("wrote", path)
