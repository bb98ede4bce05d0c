"""Whole layer steps on the GPU against the oracle, each side from the same raw inputs.

Step 1 is a synchronous warm-up on the previous step's input x' = x + 0.05 eps;
step 2 is patch i's displaced step on x against the state step 1 left.  The GPU
builds its state with its own kernels, the oracle with its own synchronous
layer: nothing crosses between them but the generator's raw inputs.
"""

import numpy as np
import pytest
import torch

import oracle
from displaced_patch_parallelism_amd import synth
from displaced_patch_parallelism_amd.configs import CONFIGS, LayerConfig
from displaced_patch_parallelism_amd.layers import DisplacedLayer
from tests.gpu_util import announce, assert_parity, gpu, host

pytestmark = pytest.mark.gpu

SMALL = {
    "c1-like": LayerConfig("c1s", "bf16", B=1, H=32, W=24, C=128, G=32, P=4, graph=("gn_silu", "conv")),
    "c2-like": LayerConfig("c2s", "bf16", B=1, H=16, W=16, C=128, G=32, P=4, graph=("gn", "attn", "conv"),
                           heads=2, head_dim=64),
    "c4b-like": LayerConfig("c4bs", "bf16", B=1, H=24, W=20, C=192, G=32, P=8, graph=("gn", "attn"),
                            heads=3, head_dim=64),
    "batched": LayerConfig("b2", "bf16", B=2, H=8, W=16, C=64, G=8, P=2, graph=("gn_silu", "conv", "attn"),
                           heads=1, head_dim=64),
    # learned Q/K/V/O projections: the K/V cache is the previous step's projected maps
    "c2p-like": LayerConfig("c2ps", "bf16", B=1, H=16, W=16, C=128, G=32, P=4,
                            graph=("gn", "attn_proj", "conv"), heads=2, head_dim=64),
    "c4bp-like": LayerConfig("c4bps", "bf16", B=1, H=24, W=20, C=192, G=32, P=8, graph=("gn", "attn_proj"),
                             heads=3, head_dim=64),
    "batched-proj": LayerConfig("b2p", "bf16", B=2, H=8, W=16, C=64, G=8, P=2,
                                graph=("gn_silu", "attn_proj", "conv"), heads=1, head_dim=64),
    "f32-proj": LayerConfig("f32p", "f32", B=1, H=8, W=12, C=64, G=8, P=2, graph=("gn", "attn_proj"),
                            heads=2, head_dim=32),
}


def two_step(c, seed=0, patches=None):
    inp = synth.layer_inputs(c, seed)
    params = {"G": c.G, "eps": c.eps, "heads": c.heads, "convs": inp.convs, "projs": inp.projs}
    layer = DisplacedLayer(c, inp.convs, projs=inp.projs)
    announce("layer warm-up", c.name)
    warm = layer.warmup(gpu(inp.x_prev, c.dtype))
    sync_outs, state = oracle.sync_layer(c.graph, params, inp.x_prev, c.P)
    for k, (g, r) in enumerate(zip(warm, sync_outs)):
        assert_parity(host(g), r, c.dtype, f"{c.name} warm-up step {k} ({c.graph[k]})")
    patches = range(c.P) if patches is None else patches
    h = c.h
    for i in patches:
        announce("layer displaced", c.name, "patch", i)
        xb = inp.x[:, i * h:(i + 1) * h]
        outs = layer.step(gpu(xb, c.dtype), i, update_state=False)
        ref_outs, _ = oracle.displaced_layer(c.graph, params, xb, state, c.P, i)
        for k, (g, r) in enumerate(zip(outs, ref_outs)):
            assert_parity(host(g), r, c.dtype, f"{c.name} patch {i} step {k} ({c.graph[k]})")
    return layer, inp, params, state


def test_c0_two_steps_all_patches():
    two_step(CONFIGS["c0"])


@pytest.mark.parametrize("name", list(SMALL))
def test_small_graphs(name):
    two_step(SMALL[name], seed=1)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c2p"])
def test_config_layers_measured_patch(name):
    c = CONFIGS[name]
    two_step(c, seed=0, patches=[c.patch])


@pytest.mark.parametrize("name", ["c2-like", "c2p-like", "batched-proj"])
def test_state_splice_matches_oracle(name):
    """After patch i's step the state holds its fresh band / moments (in place for B == 1,
    by a splice after the step otherwise); the next patch's step then reads it."""
    c = SMALL[name]
    layer, inp, params, state = two_step(c, seed=2, patches=[])
    i, h = 1, c.h
    xb = inp.x[:, i * h:(i + 1) * h]
    layer.step(gpu(xb, c.dtype), i, update_state=True)
    _, new_state = oracle.displaced_layer(c.graph, params, xb, state, c.P, i)
    torch.cuda.synchronize()
    np.testing.assert_allclose(host(layer.table), new_state["stats"], rtol=1e-4, atol=1e-4)
    for k, m in layer.maps.items():
        assert_parity(host(m), new_state["maps"][k], c.dtype, f"state map {k}")
    j = 0
    xj = inp.x[:, j * h:(j + 1) * h]
    outs = layer.step(gpu(xj, c.dtype), j, update_state=False)
    ref, _ = oracle.displaced_layer(c.graph, params, xj, new_state, c.P, j)
    for k, (g, r) in enumerate(zip(outs, ref)):
        assert_parity(host(g), r, c.dtype, f"{c.name} patch {j} after the splice, step {k}")


@pytest.mark.parametrize("name", ["c2-like", "c2p-like"])
def test_stale_equal_fresh_gives_warmup_output(name):
    """Warm-up on x itself, then a displaced step on x: equals the warm-up's band (sync)."""
    c = SMALL[name]
    inp = synth.layer_inputs(c, 3)
    layer = DisplacedLayer(c, inp.convs, projs=inp.projs)
    announce("layer stale==fresh")
    warm = layer.warmup(gpu(inp.x, c.dtype))
    for i in range(c.P):
        outs = layer.step(gpu(inp.x[:, i * c.h:(i + 1) * c.h], c.dtype), i, update_state=False)
        for k, (g, w) in enumerate(zip(outs, warm)):
            assert_parity(host(g), host(w)[:, i * c.h:(i + 1) * c.h], c.dtype, f"patch {i} step {k}")
