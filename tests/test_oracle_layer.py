"""Pins of the oracle's band splice, synchronous layer and displaced layer (CPU only).

* The synchronous layer is checked against a torch composition of
  group_norm, silu, conv2d and scaled_dot_product_attention.
* Warm-up semantics (DistriFusion summary on atlas.scime.ai, warm-up rows of
  "Measured effects reported in the paper"): with stale state equal to the
  current step's, the displaced patch equals the synchronous layer's band.
* One patch gives the plain layer.
* With a perturbed previous step the displaced result moves by the order of
  the perturbation: stale context is read, and only that.
"""

import numpy as np
import pytest
import torch

import oracle
from displaced_patch_parallelism_amd import synth
from displaced_patch_parallelism_amd.configs import LayerConfig
from tests.torch_refs import conv2d_nhwc, group_norm_nhwc, sdpa_tokens, t64

GRAPHS = {
    "gn_silu-conv-attn": ("gn_silu", "conv", "attn"),
    "gn-attn-conv": ("gn", "attn", "conv"),
    "gn_silu-conv": ("gn_silu", "conv"),
    "gn-attn": ("gn", "attn"),
    "gn-attn_proj-conv": ("gn", "attn_proj", "conv"),
    "gn-attn_proj": ("gn", "attn_proj"),
    # SDXL-like blocks: a ResNet block (two GroupNorm sites, two convs, skip connection
    # added to the second conv) and a transformer block (projected attention whose output
    # projection adds the block input)
    "resnet": ("gn_silu", "conv", "gn_silu", "conv_res"),
    "transformer": ("gn", "attn_proj_res"),
    "resnet-transformer": ("gn_silu", "conv", "gn_silu", "conv_res", "gn", "attn_proj_res"),
}


def small_cfg(graph, H=8, W=6, C=8, G=4, P=4, heads=2):
    return LayerConfig("t", "f32", B=1, H=H, W=W, C=C, G=G, P=P, graph=graph,
                       heads=heads, head_dim=C // heads)


def params_of(cfg, inp):
    return {"G": cfg.G, "eps": cfg.eps, "heads": cfg.heads, "convs": inp.convs, "projs": inp.projs}


def torch_sync(graph, params, x):
    x0 = t64(x)
    h = x0
    outs = []
    convs = iter(params["convs"])
    projs = iter(params.get("projs") or [])
    for step in graph:
        if step in ("attn_proj", "attn_proj_res"):
            wq, bq, wk, bk, wv, bv, wo, bo = (t64(a) for a in next(projs))
            B, H, W, C = h.shape
            tok = h.reshape(B, H * W, C)
            lin = torch.nn.functional.linear
            a = sdpa_tokens(lin(tok, wq, bq), lin(tok, wk, bk), lin(tok, wv, bv), params["heads"])
            h = lin(a, wo, bo).reshape(B, H, W, C)
            if step == "attn_proj_res":
                h = h + x0
        elif step.startswith("gn"):
            h = group_norm_nhwc(h, params["G"], params["eps"])
            if step == "gn_silu":
                h = torch.nn.functional.silu(h)
        elif step in ("conv", "conv_res"):
            w, b = next(convs)
            h = conv2d_nhwc(h, w, b)
            if step == "conv_res":
                h = h + x0
        else:
            B, H, W, C = h.shape
            tok = h.reshape(B, H * W, C)
            h = sdpa_tokens(tok, tok, tok, params["heads"]).reshape(B, H, W, C)
        outs.append(h.numpy())
    return outs


def test_stale_update_bytes_and_canaries():
    rng = np.random.default_rng(0)
    stale = rng.standard_normal((2, 8, 3, 4)).astype(np.float32)
    patch = rng.standard_normal((2, 2, 3, 4)).astype(np.float32)
    out = oracle.stale_update(stale, patch, 4, 2)
    assert out.dtype == np.float32
    assert out[:, 4:6].tobytes() == patch.tobytes()
    assert out[:, :4].tobytes() == stale[:, :4].tobytes()
    assert out[:, 6:].tobytes() == stale[:, 6:].tobytes()
    with pytest.raises(ValueError):
        oracle.stale_update(stale, patch[:, :1], 4, 2)


@pytest.mark.parametrize("gname", list(GRAPHS))
def test_sync_layer_matches_torch(gname):
    cfg = small_cfg(GRAPHS[gname])
    inp = synth.layer_inputs(cfg, seed=1)
    params = params_of(cfg, inp)
    outs, state = oracle.sync_layer(cfg.graph, params, inp.x, cfg.P)
    for a, b in zip(outs, torch_sync(cfg.graph, params, inp.x)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    # the state holds every band's moments of each GroupNorm input (one table per GroupNorm
    # step) and each consumer's full input map
    assert set(state["stats"]) == {k for k, s in enumerate(cfg.graph) if s in ("gn", "gn_silu")}
    for t in state["stats"].values():
        assert t.shape == (cfg.P, 1, cfg.G, 2)
    expected = {k for k, s in enumerate(cfg.graph) if s in ("conv", "conv_res", "attn")}
    expected |= {(k, kv) for k, s in enumerate(cfg.graph) if s in ("attn_proj", "attn_proj_res")
                 for kv in ("k", "v")}
    assert set(state["maps"]) == expected


@pytest.mark.parametrize("gname", list(GRAPHS))
def test_warmup_state_gives_sync_layer(gname):
    """Stale == fresh: every patch's displaced outputs equal the sync layer's band rows."""
    cfg = small_cfg(GRAPHS[gname])
    inp = synth.layer_inputs(cfg, seed=2)
    params = params_of(cfg, inp)
    sync_outs, state = oracle.sync_layer(cfg.graph, params, inp.x, cfg.P)
    h = cfg.h
    for i in range(cfg.P):
        outs, _ = oracle.displaced_layer(cfg.graph, params, inp.x[:, i * h:(i + 1) * h], state, cfg.P, i)
        for a, b in zip(outs, sync_outs):
            np.testing.assert_allclose(a, b[:, i * h:(i + 1) * h], rtol=0, atol=1e-12)


@pytest.mark.parametrize("gname", list(GRAPHS))
def test_one_patch_is_plain_layer(gname):
    cfg = small_cfg(GRAPHS[gname], P=1)
    inp = synth.layer_inputs(cfg, seed=3)
    params = params_of(cfg, inp)
    _, prev_state = oracle.sync_layer(cfg.graph, params, inp.x_prev, 1)
    outs, _ = oracle.displaced_layer(cfg.graph, params, inp.x, prev_state, 1, 0)
    for a, b in zip(outs, torch_sync(cfg.graph, params, inp.x)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


@pytest.mark.parametrize("gname", list(GRAPHS))
def test_displaced_step_reads_stale_context(gname):
    """Previous step x' = x + 0.05 eps: results differ from sync by O(0.05), not 0 and not O(1)."""
    cfg = small_cfg(GRAPHS[gname])
    inp = synth.layer_inputs(cfg, seed=4)
    params = params_of(cfg, inp)
    _, prev = oracle.sync_layer(cfg.graph, params, inp.x_prev, cfg.P)
    sync_outs, _ = oracle.sync_layer(cfg.graph, params, inp.x, cfg.P)
    i, h = 1, cfg.h
    outs, new_state = oracle.displaced_layer(cfg.graph, params, inp.x[:, i * h:(i + 1) * h], prev, cfg.P, i)
    ref = sync_outs[-1][:, i * h:(i + 1) * h]
    err = np.linalg.norm(outs[-1] - ref) / np.linalg.norm(ref)
    assert 1e-4 < err < 0.2, err
    # the new state carries the fresh band and the fresh statistics of patch i: the first
    # GroupNorm step's table gets the moments of the layer input's band
    k0 = min(new_state["stats"])
    np.testing.assert_array_equal(new_state["stats"][k0][i],
                                  oracle.gn_band_stats(inp.x[:, i * h:(i + 1) * h], cfg.G))
    for k, t in new_state["stats"].items():
        gin = inp.x[:, i * h:(i + 1) * h] if k == 0 else outs[k - 1]
        np.testing.assert_array_equal(t[i], oracle.gn_band_stats(gin, cfg.G))
        for j in range(cfg.P):
            if j != i:
                np.testing.assert_array_equal(t[j], prev["stats"][k][j])
    for k, m in new_state["maps"].items():
        np.testing.assert_array_equal(m[:, :i * h], prev["maps"][k][:, :i * h])
        np.testing.assert_array_equal(m[:, (i + 1) * h:], prev["maps"][k][:, (i + 1) * h:])


def test_all_patches_displaced_converge_to_sync():
    """Two steps of the c0 graph: a displaced step after a warm-up on x' stays near sync(x)."""
    cfg = small_cfg(GRAPHS["gn_silu-conv-attn"], H=8, W=8, C=8, G=2, P=2, heads=1)
    inp = synth.layer_inputs(cfg, seed=5)
    params = params_of(cfg, inp)
    _, prev = oracle.sync_layer(cfg.graph, params, inp.x_prev, cfg.P)
    sync_outs, _ = oracle.sync_layer(cfg.graph, params, inp.x, cfg.P)
    full = np.concatenate([oracle.displaced_layer(cfg.graph, params, inp.x[:, 4 * i:4 * i + 4], prev, 2, i)[0][-1]
                           for i in range(2)], axis=1)
    err = np.linalg.norm(full - sync_outs[-1]) / np.linalg.norm(sync_outs[-1])
    assert err < 0.1


@pytest.mark.parametrize("gname", list(GRAPHS))
def test_step_all_with_current_state_is_sync(gname):
    """All patches displaced against the current step's own (synchronous) state give the
    synchronous layer, and the next state they leave is that state again."""
    cfg = small_cfg(GRAPHS[gname])
    inp = synth.layer_inputs(cfg, seed=11)
    params = params_of(cfg, inp)
    sync_outs, state = oracle.sync_layer(cfg.graph, params, inp.x, cfg.P)
    outs, nxt = oracle.displaced_step_all(cfg.graph, params, inp.x, state, cfg.P)
    for k, (o, r) in enumerate(zip(outs, sync_outs)):
        np.testing.assert_allclose(o, r, rtol=1e-11, atol=1e-11, err_msg=f"step {k}")
    assert set(nxt["stats"]) == set(state["stats"])
    for k in state["stats"]:
        np.testing.assert_allclose(nxt["stats"][k], state["stats"][k], rtol=1e-12, atol=1e-12)
    for k in state["maps"]:
        np.testing.assert_allclose(nxt["maps"][k], state["maps"][k], rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("gname", list(GRAPHS))
def test_step_all_one_patch_is_plain_layer(gname):
    """P = 1: nothing stale is ever read, whatever the state holds."""
    cfg = small_cfg(GRAPHS[gname], P=1)
    inp = synth.layer_inputs(cfg, seed=12)
    params = params_of(cfg, inp)
    _, prev = oracle.sync_layer(cfg.graph, params, inp.x_prev, cfg.P)
    outs, _ = oracle.displaced_step_all(cfg.graph, params, inp.x, prev, cfg.P)
    ref = torch_sync(cfg.graph, params, inp.x)
    for k, (o, r) in enumerate(zip(outs, ref)):
        np.testing.assert_allclose(o, r, rtol=1e-10, atol=1e-10, err_msg=f"step {k}")


def test_step_all_next_state_is_gathered_fresh_inputs():
    """The next state holds every band's fresh moments of the GroupNorm input and every
    conv/attention step's full (gathered) input."""
    cfg = small_cfg(GRAPHS["gn_silu-conv-attn"])
    inp = synth.layer_inputs(cfg, seed=13)
    params = params_of(cfg, inp)
    _, prev = oracle.sync_layer(cfg.graph, params, inp.x_prev, cfg.P)
    outs, nxt = oracle.displaced_step_all(cfg.graph, params, inp.x, prev, cfg.P)
    np.testing.assert_allclose(nxt["stats"][0], oracle.band_moments(inp.x, cfg.G, cfg.P), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(nxt["maps"][1], outs[0])
    np.testing.assert_array_equal(nxt["maps"][2], outs[1])
    # and it differs from the previous state (the step did advance it)
    assert np.abs(nxt["maps"][1] - prev["maps"][1]).max() > 1e-3



def test_linear_brute_force():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((2, 3, 5))
    w = rng.standard_normal((4, 5))
    b = rng.standard_normal(4)
    y = oracle.linear(x, w, b)
    for i in range(2):
        for j in range(3):
            for n in range(4):
                ref = b[n]
                for k in range(5):
                    ref += x[i, j, k] * w[n, k]
                assert abs(y[i, j, n] - ref) < 1e-12
    np.testing.assert_array_equal(oracle.linear(x, w), oracle.linear(x, w, np.zeros(4)))


@pytest.mark.parametrize("P,i", [(4, 1), (2, 0)])
def test_identity_projections_reduce_to_plain_attention(P, i):
    """W = I, b = 0 for Q, K, V and O: the projected step is the unprojected one, and the
    K and V it caches are the input map itself."""
    cfg = small_cfg(("gn", "attn"), P=P)
    inp = synth.layer_inputs(cfg, seed=22)
    eye, zero = np.eye(cfg.C), np.zeros(cfg.C)
    params = params_of(cfg, inp)
    pparams = dict(params, projs=[(eye, zero) * 4])
    pgraph = ("gn", "attn_proj")
    _, prev = oracle.sync_layer(cfg.graph, params, inp.x_prev, P)
    _, pprev = oracle.sync_layer(pgraph, pparams, inp.x_prev, P)
    np.testing.assert_allclose(pprev["maps"][(1, "k")], prev["maps"][1], rtol=0, atol=1e-15)
    np.testing.assert_allclose(pprev["maps"][(1, "v")], prev["maps"][1], rtol=0, atol=1e-15)
    h = cfg.h
    xb = inp.x[:, i * h:(i + 1) * h]
    outs, st = oracle.displaced_layer(cfg.graph, params, xb, prev, P, i)
    pouts, pst = oracle.displaced_layer(pgraph, pparams, xb, pprev, P, i)
    for a, b in zip(pouts, outs):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    np.testing.assert_allclose(pst["maps"][(1, "k")], st["maps"][1], rtol=0, atol=1e-12)


def test_two_groupnorm_sites_keep_their_own_tables():
    """A ResNet block normalises two different maps.  Each GroupNorm step reads and refreshes
    its own statistics table: swapping the two tables of a warm-up state changes the
    displaced result, and with the right tables the result is the synchronous one."""
    graph = GRAPHS["resnet"]
    cfg = small_cfg(graph)
    inp = synth.layer_inputs(cfg, seed=31)
    params = params_of(cfg, inp)
    sync_outs, state = oracle.sync_layer(graph, params, inp.x, cfg.P)
    assert set(state["stats"]) == {0, 2}
    # the two sites normalise different maps, so their moments differ
    assert np.abs(state["stats"][0] - state["stats"][2]).max() > 1e-3
    i, h = 1, cfg.h
    xb = inp.x[:, i * h:(i + 1) * h]
    outs, _ = oracle.displaced_layer(graph, params, xb, state, cfg.P, i)
    np.testing.assert_allclose(outs[-1], sync_outs[-1][:, i * h:(i + 1) * h], rtol=0, atol=1e-12)
    swapped = dict(state, stats={0: state["stats"][2], 2: state["stats"][0]})
    bad, _ = oracle.displaced_layer(graph, params, xb, swapped, cfg.P, i)
    assert np.abs(bad[-1] - outs[-1]).max() > 1e-3


@pytest.mark.parametrize("gname", ["resnet", "transformer"])
def test_block_residual_is_the_block_input(gname):
    """The residual steps add the layer's own input: subtracting it leaves the plain step."""
    graph = GRAPHS[gname]
    plain = tuple(s.replace("_res", "") for s in graph)
    cfg = small_cfg(graph)
    inp = synth.layer_inputs(cfg, seed=32)
    params = params_of(cfg, inp)
    _, prev = oracle.sync_layer(graph, params, inp.x_prev, cfg.P)
    i, h = 2, cfg.h
    xb = inp.x[:, i * h:(i + 1) * h]
    outs, _ = oracle.displaced_layer(graph, params, xb, prev, cfg.P, i)
    pouts, _ = oracle.displaced_layer(plain, params, xb, prev, cfg.P, i)
    np.testing.assert_allclose(outs[-1] - xb, pouts[-1], rtol=0, atol=1e-12)
    for a, b in zip(outs[:-1], pouts[:-1]):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("gname", list(GRAPHS))
def test_state_only_sync_layer_gives_the_same_state(gname):
    """The state-only synchronous pass (used for workloads whose full attention is too large
    for the oracle) records exactly the state of the full pass."""
    cfg = small_cfg(GRAPHS[gname])
    inp = synth.layer_inputs(cfg, seed=33)
    params = params_of(cfg, inp)
    outs, state = oracle.sync_layer(cfg.graph, params, inp.x, cfg.P)
    outs2, state2 = oracle.sync_layer(cfg.graph, params, inp.x, cfg.P, state_only=True)
    assert len(outs2) == len(outs) - 1
    for a, b in zip(outs2, outs):
        np.testing.assert_array_equal(a, b)
    assert set(state2["stats"]) == set(state["stats"]) and set(state2["maps"]) == set(state["maps"])
    for k in state["stats"]:
        np.testing.assert_array_equal(state2["stats"][k], state["stats"][k])
    for k in state["maps"]:
        np.testing.assert_array_equal(state2["maps"][k], state["maps"][k])
