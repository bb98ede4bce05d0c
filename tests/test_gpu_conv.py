"""dp_conv3x3_halo on the GPU against the oracle, per call, on identical inputs."""

import itertools

import numpy as np
import pytest
import torch

import bench
import displaced_patch_parallelism_amd as dp
import oracle
from displaced_patch_parallelism_amd import synth
from displaced_patch_parallelism_amd.configs import CONFIGS
from tests.gpu_util import announce, assert_parity, gpu, host

pytestmark = pytest.mark.gpu


def conv_kernel(B, H, W, cin, cout, P, dtype="bf16"):
    """The main kernel the library's plan picks for this conv (bench.kernel_name's copy of it)."""
    from types import SimpleNamespace
    cfg = SimpleNamespace(dtype=dtype, B=B, h=H // P, W=W, C=cin)
    return bench.kernel_name("conv", cfg, cout)


def run_case(B, H, W, cin, cout, P, i, dtype, seed=0, bias=True, residual=False):
    """Both entry points (plain weights; for bf16 also the packed layout) against the oracle; the
    packed call must give bitwise the plain call's output.  With ``residual`` the residual entry
    point adds a seeded [B][h][W][Cout] map, on plain and packed weights."""
    case = synth.conv_case(B, H, W, cin, cout, dtype, seed)
    h = H // P
    xb = case.fresh[:, i * h:(i + 1) * h]
    b = case.bias if bias else None
    ref = oracle.conv3x3_halo(xb, case.stale, case.w, b, P, i)
    patch = dp.Patch(B, H, W, cin, P, i)
    xg, sg, wg = gpu(xb, dtype), gpu(case.stale, dtype), gpu(case.w, dtype)
    bg = None if b is None else gpu(b, "f32")
    what = f"conv {dtype} B{B} {H}x{W} {cin}->{cout} P{P} i{i}"
    if residual:
        rng = np.random.default_rng(seed + 1000)
        r = synth.to_storage(rng.standard_normal((B, h, W, cout), dtype=np.float32), dtype)
        rg = gpu(r, dtype)
        y = dp.dp_conv3x3_halo_residual(patch, xg, sg, wg, bg, rg)
        torch.cuda.synchronize()
        assert_parity(host(y), ref + r, dtype, what + " + residual")
        if dtype == "bf16":
            yp = dp.dp_conv3x3_halo_residual(patch, xg, sg, dp.dp_conv3x3_pack_weights(wg), bg, rg)
            torch.cuda.synchronize()
            assert torch.equal(yp.view(torch.int16), y.view(torch.int16)), "packed-weight residual conv differs"
        return y
    y = dp.dp_conv3x3_halo(patch, xg, sg, wg, bg)
    torch.cuda.synchronize()
    assert_parity(host(y), ref, dtype, what)
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


CONV_SHAPES = sorted({(c.B, c.H, c.W, c.C, c.P, c.patch, c.dtype) for c in CONFIGS.values() if c.has_conv})


@pytest.mark.parametrize("shape", CONV_SHAPES, ids=lambda s: "x".join(map(str, s[:5])) + s[6])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_config_shapes(shape, seed):
    B, H, W, C, P, ip, dtype = shape
    patches = [0, ip, P - 1] if P > 2 else list(range(P))
    for i in patches:
        announce("conv", shape, "patch", i, "seed", seed)
        run_case(B, H, W, C, C, P, i, dtype, seed=10 * seed + i)


@pytest.mark.parametrize("B,H,W,cin,cout,P,kernel", [
    (1, 32, 64, 128, 128, 4, "conv3x3_bf16_halo_wave8_kernel"),     # 64x80 tiles, K split
    (1, 128, 128, 320, 320, 4, "conv3x3_bf16_halo_wave8_kernel"),   # the c1r ResNet block's shape
    (2, 24, 1152, 64, 320, 2, "conv3x3_bf16_halo_tile_kernel"),      # 128x160 tiles
    (1, 124, 500, 64, 288, 2, "conv3x3_bf16_halo_tile_kernel"),      # 128x160 tiles, ragged rows, N tail
])
def test_residual_bf16(B, H, W, cin, cout, P, kernel):
    """The skip connection is added before rounding in every kernel's epilogue (and in the
    split-K reduction)."""
    assert conv_kernel(B, H, W, cin, cout, P) == kernel
    for i in sorted({0, 1, P - 1}):
        announce("conv residual", B, H, W, cin, cout, P, i, kernel)
        run_case(B, H, W, cin, cout, P, i, "bf16", seed=40 + i, residual=True)


def test_residual_f32():
    for i in range(2):
        announce("conv residual f32", i)
        run_case(2, 8, 4, 8, 5, 2, i, "f32", seed=50 + i, residual=True)


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
    # 128x160 tiles (4 rows): 62 = 15*4 + 2 rows, 500 = 15*32 + 20 columns, 288 = 160 + 128
    (1, 124, 500, 64, 288, 2),
    (2, 96, 254, 64, 320, 2),   # over two batch images, ragged columns
    (2, 24, 1152, 64, 320, 2),  # 12-row bands, 36 column tiles
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


ONEHOT_SHAPES = [
    # (B, H, W, C, P, dtype, kernel the plan picks)
    (1, 8, 9, 64, 4, "bf16", "conv3x3_bf16_halo_wave8_kernel"),
    (1, 240, 480, 64, 2, "bf16", "conv3x3_bf16_halo_tile_kernel"),
    (2, 24, 1152, 320, 2, "bf16", "conv3x3_bf16_halo_tile_kernel"),
    (1, 8, 9, 8, 4, "f32", "conv3x3_f32_direct_kernel"),
]


@pytest.mark.parametrize("B,H,W,C,P,dtype,kernel", ONEHOT_SHAPES)
def test_onehot_halo_indexing_bit_exact(B, H, W, C, P, dtype, kernel):
    """One-hot weights copy one tap: fresh values are negative, stale positive, so
    the output names which buffer (or the zero padding) every source came from.  Run on
    every kernel the plan can pick (the small-map and the large-map tile kernels, f32; the
    256x160 tiles, used only with a GroupNorm folded in, are bitwise equal to the unfused
    calls in test_gpu_gn_conv)."""
    assert conv_kernel(B, H, W, C, C, P, dtype) == kernel
    rng = np.random.default_rng(7)
    fresh = -rng.integers(1, 101, size=(B, H, W, C)).astype(np.float32)
    stale = rng.integers(1, 101, size=(B, H, W, C)).astype(np.float32)
    h = H // P
    sg = gpu(stale, dtype)
    for i, (ky, kx) in itertools.product(range(P), itertools.product(range(3), range(3))):
        announce("conv one-hot", (B, H, W, C, P), kernel, "patch", i, "tap", ky, kx)
        w = np.zeros((C, 3, 3, C), np.float32)
        w[np.arange(C), ky, kx, np.arange(C)] = 1.0
        xb = fresh[:, i * h:(i + 1) * h]
        ref = oracle.conv3x3_halo(xb, stale, w, None, P, i)
        y = dp.dp_conv3x3_halo(dp.Patch(B, H, W, C, P, i), gpu(xb, dtype), sg, gpu(w, dtype))
        got = host(y)
        assert np.array_equal(got, ref), f"patch {i} tap ({ky},{kx})"


@pytest.mark.parametrize("B,H,W,C,P,i,kernel", [
    (1, 64, 64, 640, 4, 1, "conv3x3_bf16_halo_wave8_kernel"),     # c2 (K split)
    (1, 240, 480, 64, 2, 1, "conv3x3_bf16_halo_tile_kernel"),
    (1, 480, 480, 320, 8, 1, "conv3x3_bf16_halo_tile_kernel"),    # c4a
    (2, 24, 1152, 320, 2, 0, "conv3x3_bf16_halo_tile_kernel"),
])
def test_determinism_and_stale_rows_only(B, H, W, C, P, i, kernel):
    """Repeated calls are bitwise equal, and rows of the stale map other than r0-1 and r0+h
    are never read: poisoning every other stale row (band i included) leaves the output's
    bits unchanged."""
    assert conv_kernel(B, H, W, C, C, P) == kernel
    announce("conv determinism", (B, H, W, C, P, i), kernel)
    case = synth.conv_case(B, H, W, C, C, "bf16", 3)
    h = H // P
    r0 = i * h
    p = dp.Patch(B, H, W, C, P, i)
    xb, st = gpu(case.fresh[:, r0:r0 + h], "bf16"), gpu(case.stale, "bf16")
    w, b = gpu(case.w, "bf16"), gpu(case.bias, "f32")
    y1 = dp.dp_conv3x3_halo(p, xb, st, w, b)
    y2 = dp.dp_conv3x3_halo(p, xb, st, w, b)
    st2 = st.clone()
    if r0 - 1 > 0:
        st2[:, :r0 - 1] = 1000.0
    st2[:, r0 + h + 1:] = -1000.0
    st2[:, r0:r0 + h] = 77.0
    y3 = dp.dp_conv3x3_halo(p, xb, st2, w, b)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))
