"""dp_conv3x3_halo on the GPU against the oracle, per call, on identical inputs."""

import itertools

import numpy as np
import pytest
import torch

import displaced_patch_parallelism_amd as dp
import oracle
from displaced_patch_parallelism_amd import synth
from displaced_patch_parallelism_amd.configs import CONFIGS
from tests.gpu_util import announce, assert_parity, gpu, host

pytestmark = pytest.mark.gpu


def run_case(B, H, W, cin, cout, P, i, dtype, seed=0, bias=True):
    """Both entry points (plain weights; for bf16 also the packed layout) against the oracle; the
    packed call must give bitwise the plain call's output."""
    case = synth.conv_case(B, H, W, cin, cout, dtype, seed)
    h = H // P
    xb = case.fresh[:, i * h:(i + 1) * h]
    b = case.bias if bias else None
    ref = oracle.conv3x3_halo(xb, case.stale, case.w, b, P, i)
    patch = dp.Patch(B, H, W, cin, P, i)
    xg, sg, wg = gpu(xb, dtype), gpu(case.stale, dtype), gpu(case.w, dtype)
    bg = None if b is None else gpu(b, "f32")
    y = dp.dp_conv3x3_halo(patch, xg, sg, wg, bg)
    torch.cuda.synchronize()
    assert_parity(host(y), ref, dtype, f"conv {dtype} B{B} {H}x{W} {cin}->{cout} P{P} i{i}")
    if dtype == "bf16":
        yp = dp.dp_conv3x3_halo_packed(patch, xg, sg, dp.dp_conv3x3_pack_weights(wg), bg)
        torch.cuda.synchronize()
        assert torch.equal(yp.view(torch.int16), y.view(torch.int16)), "packed-weight conv differs"
    return y


@pytest.mark.parametrize("cin,cout", [(64, 32), (320, 320), (128, 352)])
def test_pack_weights_layout(cin, cout):
    """w_packed[ky][ci // 32][kx][co][ci % 32] = w[co][ky][kx][ci], bit for bit."""
    rng = np.random.default_rng(cin + cout)
    w = rng.standard_normal((cout, 3, 3, cin), dtype=np.float32)
    wg = gpu(w, "bf16")
    wp = dp.dp_conv3x3_pack_weights(wg)
    torch.cuda.synchronize()
    bits = wg.view(torch.int16).cpu().numpy()
    expect = bits.reshape(cout, 3, 3, cin // 32, 32).transpose(1, 3, 2, 0, 4)
    assert np.array_equal(wp.view(torch.int16).cpu().numpy(), expect)


@pytest.mark.parametrize("name", [n for n, c in CONFIGS.items() if c.has_conv])
def test_config_shapes(name):
    c = CONFIGS[name]
    patches = [0, c.patch, c.P - 1] if c.P > 2 else list(range(c.P))
    for i in patches:
        announce("conv", name, "patch", i)
        run_case(c.B, c.H, c.W, c.C, c.C, c.P, i, c.dtype, seed=10 + i)


@pytest.mark.parametrize("B,H,W,cin,cout,P", [
    (1, 12, 7, 64, 32, 3),      # ragged M (h*W = 28), one partial N tile
    (2, 8, 10, 128, 96, 2),     # batch 2 across a tile, N tail inside a 160 tile
    (1, 6, 33, 192, 352, 2),    # ragged W, N = 2 tiles + 32
    (1, 4, 16, 64, 64, 4),      # one-row bands: both halos from the stale map
])
def test_ragged_bf16(B, H, W, cin, cout, P):
    for i in range(P):
        announce("conv ragged", B, H, W, cin, cout, P, i)
        run_case(B, H, W, cin, cout, P, i, "bf16", seed=i)


@pytest.mark.parametrize("B,H,W,cin,cout,P", [
    # 256x160 tiles (8 rows): 62 = 7*8 + 6 rows, 500 = 15*32 + 20 columns, 288 = 160 + 128
    (1, 124, 500, 64, 288, 2),
    (2, 96, 254, 64, 320, 2),   # 256x160 tiles over two batch images, ragged columns
    # 128x160 tiles (4 rows): 12-row bands need a second round of 8-row tiles
    (2, 24, 1152, 64, 320, 2),
])
def test_large_map_tiles_bf16(B, H, W, cin, cout, P):
    for i in range(P):
        announce("conv large-map tiles", B, H, W, cin, cout, P, i)
        run_case(B, H, W, cin, cout, P, i, "bf16", seed=20 + i)


@pytest.mark.parametrize("B,H,W,cin,cout,P", [(1, 6, 5, 3, 4, 3), (2, 8, 4, 8, 5, 2), (1, 16, 16, 32, 32, 2)])
def test_f32(B, H, W, cin, cout, P):
    for i in range(P):
        announce("conv f32", B, H, W, cin, cout, P, i)
        run_case(B, H, W, cin, cout, P, i, "f32", seed=i, bias=i % 2 == 0)


@pytest.mark.parametrize("dtype,C", [("bf16", 64), ("f32", 8)])
def test_onehot_halo_indexing_bit_exact(dtype, C):
    """One-hot weights copy one tap: fresh values are negative, stale positive, so
    the output names which buffer (or the zero padding) every source came from."""
    B, H, W, P = 1, 8, 9, 4
    rng = np.random.default_rng(7)
    fresh = -rng.integers(1, 101, size=(B, H, W, C)).astype(np.float32)
    stale = rng.integers(1, 101, size=(B, H, W, C)).astype(np.float32)
    h = H // P
    for i, (ky, kx) in itertools.product(range(P), itertools.product(range(3), range(3))):
        w = np.zeros((C, 3, 3, C), np.float32)
        w[np.arange(C), ky, kx, np.arange(C)] = 1.0
        xb = fresh[:, i * h:(i + 1) * h]
        ref = oracle.conv3x3_halo(xb, stale, w, None, P, i)
        y = dp.dp_conv3x3_halo(dp.Patch(B, H, W, C, P, i), gpu(xb, dtype), gpu(stale, dtype), gpu(w, dtype))
        got = host(y)
        assert np.array_equal(got, ref), f"patch {i} tap ({ky},{kx})"


def test_determinism_and_stale_rows_only():
    c = CONFIGS["c2"]
    announce("conv determinism c2")
    case = synth.conv_case(1, c.H, c.W, c.C, c.C, "bf16", 3)
    i, h = 1, c.h
    p = dp.Patch(1, c.H, c.W, c.C, c.P, i)
    xb, st, w, b = gpu(case.fresh[:, h:2 * h], "bf16"), gpu(case.stale, "bf16"), gpu(case.w, "bf16"), gpu(case.bias, "f32")
    y1 = dp.dp_conv3x3_halo(p, xb, st, w, b)
    y2 = dp.dp_conv3x3_halo(p, xb, st, w, b)
    # rows of the stale map other than r0-1 and r0+h are never read
    st2 = st.clone()
    st2[:, :h - 1] = 1000.0
    st2[:, 2 * h + 1:] = -1000.0
    st2[:, h:2 * h] = 77.0
    y3 = dp.dp_conv3x3_halo(p, xb, st2, w, b)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))
