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
from tests.gpu_util import announce, assert_parity, assert_table, gpu, host

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
    # SDXL-like blocks: ResNet (two GroupNorm sites, skip added by the second conv), transformer
    # (skip added by the output projection), both in sequence; f32 and batched variants
    "resnet-like": LayerConfig("r1s", "bf16", B=1, H=32, W=24, C=128, G=32, P=4,
                               graph=("gn_silu", "conv", "gn_silu", "conv_res")),
    "transformer-like": LayerConfig("t2s", "bf16", B=1, H=16, W=16, C=128, G=32, P=4,
                                    graph=("gn", "attn_proj_res"), heads=2, head_dim=64),
    "block-like": LayerConfig("blk", "bf16", B=1, H=16, W=16, C=128, G=32, P=4,
                              graph=("gn_silu", "conv", "gn_silu", "conv_res", "gn", "attn_proj_res"),
                              heads=2, head_dim=64),
    "block-batched": LayerConfig("blk2", "bf16", B=2, H=8, W=16, C=64, G=8, P=2,
                                 graph=("gn_silu", "conv", "gn_silu", "conv_res", "gn", "attn_proj_res"),
                                 heads=1, head_dim=64),
    "block-f32": LayerConfig("blkf", "f32", B=1, H=8, W=12, C=64, G=8, P=2,
                             graph=("gn_silu", "conv", "gn_silu", "conv_res", "gn", "attn_proj_res"),
                             heads=2, head_dim=32),
    # a graph that starts with a conv: its stale map's band i is the layer input itself
    "conv-first": LayerConfig("cf", "bf16", B=1, H=16, W=16, C=128, G=32, P=4, graph=("conv", "gn", "attn"),
                              heads=2, head_dim=64),
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


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c2p", "c1r", "c2t"])
def test_config_layers_measured_patch(name):
    c = CONFIGS[name]
    two_step(c, seed=0, patches=[c.patch])


def sample_rows(c, seed, n=256):
    """A seeded sample of a band's query rows plus every band-edge row (first and last map row)."""
    rng = np.random.default_rng(seed)
    edges = list(range(c.W)) + list(range(c.Nq - c.W, c.Nq))
    return np.array(sorted(set(rng.choice(c.Nq, n, replace=False).tolist()) | set(edges)))


@pytest.mark.parametrize("name", ["c4a", "c4b", "c4bp"])
def test_3840px_layers_measured_patch(name):
    """The 3840px layers at full size: the GPU warm-up on x' and patch 1's displaced step on x
    against the oracle (its state from the synchronous pass on x', without that pass's own
    attention output, which the state never needs).  An attention that ends the graph is
    compared on a seeded sample of query rows plus every band-edge row."""
    c = CONFIGS[name]
    inp = synth.layer_inputs(c, 0)
    params = {"G": c.G, "eps": c.eps, "heads": c.heads, "convs": inp.convs, "projs": inp.projs}
    layer = DisplacedLayer(c, inp.convs, projs=inp.projs)
    announce("layer warm-up", c.name)
    layer.warmup(gpu(inp.x_prev, c.dtype))
    _, state = oracle.sync_layer(c.graph, params, inp.x_prev, c.P, state_only=True)
    i, h = c.patch, c.h
    xb = inp.x[:, i * h:(i + 1) * h]
    announce("layer displaced", c.name, "patch", i)
    outs = layer.step(gpu(xb, c.dtype), i, update_state=False)
    torch.cuda.synchronize()
    last = c.graph[-1]
    if last in ("conv", "conv_res"):
        ref, _ = oracle.displaced_layer(c.graph, params, xb, state, c.P, i)
        for k, (g, r) in enumerate(zip(outs, ref)):
            assert_parity(host(g), r, c.dtype, f"{c.name} patch {i} step {k} ({c.graph[k]})")
        return
    head = c.graph[:-1]
    step_of = lambda key: key[0] if isinstance(key, tuple) else key  # noqa: E731
    sub = {"stats": {k: t for k, t in state["stats"].items() if k < len(head)},
           "maps": {k: m for k, m in state["maps"].items() if step_of(k) < len(head)}}
    ref_head, _ = oracle.displaced_layer(head, params, xb, sub, c.P, i)
    for k, (g, r) in enumerate(zip(outs, ref_head)):
        assert_parity(host(g), r, c.dtype, f"{c.name} patch {i} step {k} ({c.graph[k]})")
    rows = sample_rows(c, seed=1)
    k = len(c.graph) - 1
    tok = ref_head[-1].reshape(c.B, c.Nq, c.C)
    if last == "attn":
        st = np.asarray(state["maps"][k]).reshape(c.B, c.N, c.C)
        ref = oracle.attention_splice(tok, tok, tok, st, st, c.H, c.W, c.P, i, c.heads, rows=rows)
    else:
        wq, bq, wk, bk, wv, bv, wo, bo = inp.projs[0]
        q, kk, vv = oracle.linear(tok, wq, bq), oracle.linear(tok, wk, bk), oracle.linear(tok, wv, bv)
        ks = np.asarray(state["maps"][(k, "k")]).reshape(c.B, c.N, c.C)
        vs = np.asarray(state["maps"][(k, "v")]).reshape(c.B, c.N, c.C)
        a = oracle.attention_splice(q, kk, vv, ks, vs, c.H, c.W, c.P, i, c.heads, rows=rows)
        ref = oracle.linear(a, wo, bo)
        if last == "attn_proj_res":
            ref = ref + xb.reshape(c.B, c.Nq, c.C)[:, rows]
    got = host(outs[-1]).reshape(c.B, c.Nq, c.C)[:, rows]
    assert_parity(got, ref, c.dtype, f"{c.name} patch {i} step {k} ({last}), {len(rows)} sampled rows")


@pytest.mark.parametrize("name", ["c2-like", "c2p-like", "batched-proj", "conv-first", "block-like",
                                  "block-batched"])
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
    for k, tab in layer.tables.items():
        assert_table(host(tab), new_state["stats"][k], c.dtype, k, f"statistics table {k}")
    for k, m in layer.maps.items():
        assert_parity(host(m), new_state["maps"][k], c.dtype, f"state map {k}")
    j = 0
    xj = inp.x[:, j * h:(j + 1) * h]
    outs = layer.step(gpu(xj, c.dtype), j, update_state=False)
    ref, _ = oracle.displaced_layer(c.graph, params, xj, new_state, c.P, j)
    for k, (g, r) in enumerate(zip(outs, ref)):
        assert_parity(host(g), r, c.dtype, f"{c.name} patch {j} after the splice, step {k}")


@pytest.mark.parametrize("name", ["c2-like", "c2p-like", "block-like"])
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


FUSE_CASES = {
    "c4a": CONFIGS["c4a"],                 # GroupNorm folded into the 256x160-tile conv
    "c1r": CONFIGS["c1r"],                 # small-map ResNet block: three kernels inside the call
    # a ResNet block on 256x160 tiles: both GroupNorm sites folded, the second conv adding the skip
    "resnet-tile8": LayerConfig("r8", "bf16", B=1, H=192, W=512, C=128, G=32, P=2,
                                graph=("gn_silu", "conv", "gn_silu", "conv_res")),
    "block-like": SMALL["block-like"],
}


@pytest.mark.parametrize("name", list(FUSE_CASES))
def test_fused_groupnorm_conv_step_equals_unfused(name):
    """A state-refreshing step with each GroupNorm -> conv pair as one dp_groupnorm_conv3x3_halo
    call gives bit for bit the outputs, stale maps and statistics tables of the step that runs
    the GroupNorm and the conv as two calls."""
    c = FUSE_CASES[name]
    inp = synth.layer_inputs(c, 4)
    i, h = c.patch, c.h
    xb = inp.x[:, i * h:(i + 1) * h]
    got = {}
    for fuse in (True, False):
        layer = DisplacedLayer(c, inp.convs, projs=inp.projs, fuse=fuse)
        announce("layer fused" if fuse else "layer unfused", c.name, "patch", i)
        layer.warmup(gpu(inp.x_prev, c.dtype))
        names = [n for n, _, _ in layer.calls(gpu(xb, c.dtype), i)]
        assert any("+" in n for n in names) == fuse, names
        outs = layer.step(gpu(xb, c.dtype), i, update_state=True)
        torch.cuda.synchronize()
        got[fuse] = ([o.clone() for o in outs], {k: m.clone() for k, m in layer.maps.items()},
                     {k: t.clone() for k, t in layer.tables.items()})
        del layer
    (of, mf, tf), (ou, mu, tu) = got[True], got[False]
    assert len(of) == len(ou) == len(c.graph)
    bitsof = lambda t: t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)  # noqa: E731
    for k, (a, b) in enumerate(zip(of, ou)):
        assert torch.equal(bitsof(a), bitsof(b)), f"{name} step {k} ({c.graph[k]})"
    for k in mu:
        assert torch.equal(bitsof(mf[k]), bitsof(mu[k])), f"{name} stale map {k}"
    for k in tu:
        assert torch.equal(tf[k], tu[k]), f"{name} statistics table {k}"


def test_fused_resnet_block_state_matches_oracle():
    """The 256x160-tile ResNet block's state-refreshing step (both GroupNorm sites folded into
    their convs) against the oracle: outputs, refreshed stale maps and statistics tables."""
    c = FUSE_CASES["resnet-tile8"]
    inp = synth.layer_inputs(c, 5)
    params = {"G": c.G, "eps": c.eps, "heads": c.heads, "convs": inp.convs, "projs": inp.projs}
    layer = DisplacedLayer(c, inp.convs, projs=inp.projs)
    announce("layer fused resnet vs oracle", c.name)
    layer.warmup(gpu(inp.x_prev, c.dtype))
    _, state = oracle.sync_layer(c.graph, params, inp.x_prev, c.P, state_only=True)
    i, h = 1, c.h
    xb = inp.x[:, i * h:(i + 1) * h]
    outs = layer.step(gpu(xb, c.dtype), i, update_state=True)
    torch.cuda.synchronize()
    ref, new_state = oracle.displaced_layer(c.graph, params, xb, state, c.P, i)
    for k, (g, r) in enumerate(zip(outs, ref)):
        assert_parity(host(g), r, c.dtype, f"{c.name} patch {i} step {k} ({c.graph[k]})")
    for k, tab in layer.tables.items():
        assert_table(host(tab), new_state["stats"][k], c.dtype, k, f"statistics table {k}")
    for k, m in layer.maps.items():
        assert_parity(host(m), new_state["maps"][k], c.dtype, f"state map {k}")
