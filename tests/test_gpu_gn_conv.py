"""dp_groupnorm_conv3x3_halo on the GPU.

The fused call stands for three calls: dp_groupnorm_async into a band,
dp_stale_update of that band into the conv's stale map, and the conv (with
an optional residual).  Its outputs -- the conv output, the updated stale
map and the fresh moments -- must equal theirs bit for bit, whichever path
the call takes (GroupNorm folded into the 256x160-tile conv, or the three
kernels), and they are checked against the oracle too.
"""

import numpy as np
import pytest
import torch

import bench
import displaced_patch_parallelism_amd as dp
import oracle
from displaced_patch_parallelism_amd import synth
from tests.gpu_util import announce, assert_parity, gpu, host

pytestmark = pytest.mark.gpu

MODES = {"corrected": oracle.GN_CORRECTED, "local": oracle.GN_LOCAL, "stale": oracle.GN_STALE}


def bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def fused_path(B, H, W, C, cout, P, G, dtype):
    """Whether the call folds the GroupNorm into the conv: the 256x160-tile conv, and the
    GroupNorm's lanes (normalising block threads / G) and parameter table fit that kernel."""
    from types import SimpleNamespace
    cfg = SimpleNamespace(dtype=dtype, B=B, h=H // P, W=W, C=C)
    if bench.kernel_name("gn_silu+conv", cfg, cout) != "conv3x3_bf16_gn_tile8_kernel":
        return False
    vpt = C // 8
    rows = max(1, 512 // vpt) if vpt < 512 else 1
    threads = vpt * rows
    if threads < G:
        threads = vpt * -(-G // vpt)
    lanes = threads // G
    table_off = ((lanes * G + G) * 8 + 15) & ~15
    return lanes * G <= 512 and G <= 512 and table_off + 8 * C <= 16 * 1024


def run_case(B, H, W, C, cout, G, P, i, dtype, mode="corrected", act="silu", affine=True, residual=False,
             packed=True, slot_i=True, seed=0, check_oracle=True):
    rng = np.random.default_rng(seed)
    fresh, stale_in, gamma, beta = synth.gn_case(B, H, W, C, dtype, seed, affine=affine)
    h = H // P
    xb = fresh[:, i * h:(i + 1) * h]
    table = oracle.band_moments(stale_in, G, P).astype(np.float32)       # previous step's moments
    u_prev = synth.to_storage(rng.standard_normal((B, H, W, C), dtype=np.float32), dtype)   # conv's stale map
    w, bias = synth.conv_params(rng, C, cout, dtype)
    res = synth.to_storage(rng.standard_normal((B, h, W, cout), dtype=np.float32), dtype) if residual else None
    patch = dp.Patch(B, H, W, C, P, i)
    what = f"gn+conv {dtype} B{B} {H}x{W} {C}->{cout} G{G} P{P} i{i} {mode} {act} res={residual}"
    announce(what)

    xg = gpu(xb, dtype)
    wg = gpu(w, dtype)
    wk = dp.dp_conv3x3_pack_weights(wg) if packed else wg
    bg = gpu(bias, "f32")
    ga = gpu(gamma, "f32") if gamma is not None else None
    be = gpu(beta, "f32") if beta is not None else None
    rg = gpu(res, dtype) if residual else None

    # the fused call; fresh moments into slot i of its table when asked (CORRECTED only)
    t_f = gpu(table, "f32")
    u_f = gpu(u_prev, dtype)
    st_f = t_f[i] if slot_i else torch.empty((B, G, 2), dtype=torch.float32, device=xg.device)
    y_f, _ = dp.dp_groupnorm_conv3x3_halo(patch, xg, G, u_f, wk, bg, stale_stats=t_f, mode=mode, act=act,
                                          gamma=ga, beta=be, fresh_stats_out=st_f, residual=rg, packed=packed)
    # the three calls
    t_r = gpu(table, "f32")
    u_r = gpu(u_prev, dtype)
    st_r = t_r[i] if slot_i else torch.empty((B, G, 2), dtype=torch.float32, device=xg.device)
    gn_out, _ = dp.dp_groupnorm_async(patch, xg, G, t_r, 1e-5, mode, act, ga, be, fresh_stats_out=st_r)
    dp.dp_stale_update(patch, gn_out, u_r)
    y_r = dp.dp_conv3x3_halo_residual(patch, gn_out, u_r, wk, bg, rg, packed=packed)
    torch.cuda.synchronize()

    assert torch.equal(bits(y_f), bits(y_r)), what + ": conv output differs from the three calls"
    assert torch.equal(bits(u_f), bits(u_r)), what + ": stale map differs from the three calls"
    assert torch.equal(bits(st_f), bits(st_r)), what + ": fresh moments differ from the three calls"
    if slot_i:
        assert torch.equal(bits(t_f), bits(t_r)), what + ": statistics table differs"

    if check_oracle:
        ref_gn, ref_st = oracle.gn_async(xb, table, P, i, G, 1e-5, MODES[mode], gamma, beta, act)
        u_host = host(u_f)
        assert_parity(u_host[:, i * h:(i + 1) * h], ref_gn, dtype, what + " normalised band")
        others = np.ones(H, bool)
        others[i * h:(i + 1) * h] = False
        assert np.array_equal(u_host[:, others], np.asarray(u_prev, np.float64)[:, others]), \
            what + ": rows outside band i of the stale map changed"
        np.testing.assert_allclose(host(st_f), ref_st, rtol=1e-4, atol=1e-5)
        u_ref = oracle.stale_update(u_prev, ref_gn, P, i)
        ref_y = oracle.conv3x3_halo(ref_gn, u_ref, w, bias, P, i)
        if residual:
            ref_y = ref_y + res
        assert_parity(host(y_f), ref_y, dtype, what + " conv output")
    return y_f


def test_c4a_layer_shape_fused():
    """The 3840px conv layer's shape (480x480x320, 8 bands, 32 groups, SiLU), middle and edge
    bands: the GroupNorm is folded into the 256x160-tile conv."""
    assert fused_path(1, 480, 480, 320, 320, 8, 32, "bf16")
    for i in (0, 3, 7):
        run_case(1, 480, 480, 320, 320, 32, 8, i, "bf16", seed=60 + i, check_oracle=i == 3)


@pytest.mark.parametrize("i", [0, 2, 3])
def test_batched_ragged_fused(i):
    """Two batch images, 52-row bands (6.5 tiles of 8 rows), 232 columns (7.25 tiles of 32),
    192 output channels (160 + 32): every tile edge the fused kernel has.  The workspace
    query shows the fused path (no band buffer for B = 2)."""
    B, H, W, C, cout, G, P = 2, 208, 232, 128, 192, 32, 4
    assert fused_path(B, H, W, C, cout, P, G, "bf16")
    p = dp.Patch(B, H, W, C, P, i)
    assert dp.workspace_bytes("groupnorm_conv", p, dp.DP_BF16, G, cout) == \
        dp.workspace_bytes("groupnorm", p, dp.DP_BF16, G)
    run_case(B, H, W, C, cout, G, P, i, "bf16", seed=70 + i)


@pytest.mark.parametrize("mode,act,affine,residual,packed,slot_i", [
    ("corrected", None, False, True, False, True),
    ("local", "silu", True, False, True, False),
    ("stale", None, True, True, True, False),
    ("corrected", "silu", True, True, True, False),
])
def test_modes_fused(mode, act, affine, residual, packed, slot_i):
    """Every GroupNorm mode, with and without SiLU, affine parameters, residual and packed
    weights, on the fused path."""
    B, H, W, C, cout, G, P = 2, 208, 232, 128, 192, 32, 4
    run_case(B, H, W, C, cout, G, P, 1, "bf16", mode=mode, act=act, affine=affine, residual=residual,
             packed=packed, slot_i=slot_i, seed=80)


@pytest.mark.parametrize("B,H,W,C,cout,G,P,dtype", [
    (1, 64, 64, 320, 320, 32, 4, "bf16"),     # small map: the K-split conv, GroupNorm in place
    (2, 24, 40, 64, 96, 8, 2, "bf16"),        # B = 2: GroupNorm into the workspace, then spliced
    (2, 8, 6, 16, 12, 4, 2, "f32"),           # fp32
])
def test_unfused_shapes(B, H, W, C, cout, G, P, dtype):
    """Shapes the fused kernel does not take run the three kernels inside the call."""
    assert not fused_path(B, H, W, C, cout, P, G, dtype)
    for i in sorted({0, P - 1}):
        run_case(B, H, W, C, cout, G, P, i, dtype, residual=i == 0, packed=dtype == "bf16", seed=90 + i)

