"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects invalid arguments on the host before touching the GPU runtime.

No call here reaches a kernel launch: every case fails validation first.
"""

import ctypes
import os
import re

import pytest

import displaced_patch_parallelism_amd as dp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dp.h")



def test_library_is_built():
    """The boundary suite needs the built library; a missing one is a failure, not a skip."""
    assert os.path.exists(dp.LIB_PATH), f"{dp.LIB_PATH} is not built (run __graft_entry__.build())"


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dp_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert {"dp_groupnorm_async", "dp_conv3x3_halo", "dp_attention_splice", "dp_stale_update"} <= set(names)
    lib = dp.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert dp.version().startswith("dp ")


P_OK = dp.Patch(1, 16, 8, 64, 4, 1)
FAKE = 0x10000          # 16-byte aligned, never dereferenced: validation fails first
FAKE2 = 0x20000000


def call_stale(p, dtype=dp.DP_BF16, x=FAKE, s=FAKE2):
    return dp.lib().dp_stale_update(dp._cpatch(p), dtype, x, s, None)


@pytest.mark.parametrize("p,msg", [
    (dp.Patch(1, 10, 8, 64, 4, 0), "divisible"),
    (dp.Patch(1, 16, 8, 64, 4, 4), "patch index"),
    (dp.Patch(1, 16, 8, 64, 4, -1), "patch index"),
    (dp.Patch(0, 16, 8, 64, 4, 0), ">= 1"),
    (dp.Patch(1, 16, 0, 64, 4, 0), ">= 1"),
])
def test_bad_geometry(p, msg):
    assert call_stale(p) == dp.DP_ERR_ARG
    assert msg in dp.lib().dp_last_error().decode()


def test_null_and_misaligned_pointers():
    assert call_stale(P_OK, x=0) == dp.DP_ERR_ARG
    assert "NULL" in dp.lib().dp_last_error().decode()
    assert call_stale(P_OK, x=FAKE + 2) == dp.DP_ERR_ARG
    assert "aligned" in dp.lib().dp_last_error().decode()
    assert call_stale(P_OK, dtype=7) == dp.DP_ERR_ARG


def test_stale_update_overlap_rejected():
    # x_patch inside the map but not band i
    assert call_stale(P_OK, x=FAKE2 + 16, s=FAKE2) == dp.DP_ERR_ARG
    assert "overlap" in dp.lib().dp_last_error().decode()


def test_stale_update_in_place_is_noop():
    # x_patch == band i of stale: nothing to do, succeeds without touching memory
    band_off = P_OK.r0 * P_OK.W * P_OK.C * 2
    assert call_stale(P_OK, x=FAKE2 + band_off, s=FAKE2) == dp.DP_OK


def ws_query(kind, p, dtype, *args):
    out = ctypes.c_size_t(123)
    fn = {"gn": dp.lib().dp_groupnorm_async_ws, "conv": dp.lib().dp_conv3x3_halo_ws,
          "attn": dp.lib().dp_attention_splice_ws}[kind]
    st = fn(dp._cpatch(p), dtype, *args, ctypes.byref(out))
    return st, out.value


def test_workspace_queries():
    st, n = ws_query("gn", dp.Patch(1, 128, 128, 320, 4, 1), dp.DP_BF16, 32)
    assert st == dp.DP_OK and n > 0
    st, n = ws_query("conv", dp.Patch(1, 480, 480, 320, 8, 1), dp.DP_BF16, 320)
    assert st == dp.DP_OK
    st, n = ws_query("conv", dp.Patch(1, 32, 32, 1280, 8, 1), dp.DP_BF16, 1280)
    assert st == dp.DP_OK and n > 0          # small M: split along K
    st, n = ws_query("attn", dp.Patch(1, 64, 64, 640, 4, 1), dp.DP_BF16, 10, 64)
    assert st == dp.DP_OK and n > 0          # few query tiles: split along keys
    st, n = ws_query("attn", dp.Patch(1, 16, 16, 32, 2, 1), dp.DP_F32, 1, 32)
    assert st == dp.DP_OK and n == 0


@pytest.mark.parametrize("kind,p,args,expect", [
    # conv: fp32 partials, one [M][Cout] slab per K split; 64x80 tiles split along K until ~256
    # workgroups run: c2 has 16 x 8 = 128 tiles -> 2 splits, c3 2 x 16 = 32 tiles -> 8
    ("conv", dp.Patch(1, 64, 64, 640, 4, 1), (640,), 2 * 1024 * 640 * 4),
    ("conv", dp.Patch(1, 32, 32, 1280, 8, 1), (1280,), 8 * 128 * 1280 * 4),
    ("conv", dp.Patch(1, 128, 128, 320, 4, 1), (320,), 0),       # 256 tiles: no split
    ("conv", dp.Patch(1, 480, 480, 320, 8, 1), (320,), 0),       # large-map tiles: no split
    # attention: per key split, fp32 O [heads][Nq][64] and (max, sum) per query; 256-query
    # tiles x heads, split to fill whole rounds of workgroups (256, or 512 for grids of 512 or
    # more: two per CU): c2 40 units -> 6, c3 20 -> 8, c4b 290 -> 7
    ("attn", dp.Patch(1, 64, 64, 640, 4, 1), (10, 64), 6 * 10 * 1024 * (64 * 4 + 8)),
    ("attn", dp.Patch(1, 32, 32, 1280, 8, 1), (20, 64), 8 * 20 * 128 * (64 * 4 + 8)),
    ("attn", dp.Patch(1, 240, 240, 640, 8, 1), (10, 64), 7 * 10 * 7200 * (64 * 4 + 8)),
    # GroupNorm: (sum, sum of squares) per statistics block and group; c1 splits its 4096 tokens
    # into 228 blocks of 18
    ("gn", dp.Patch(1, 128, 128, 320, 4, 1), (32,), 228 * 32 * 2 * 4),
])
def test_workspace_sizes_follow_the_launch_plans(kind, p, args, expect):
    st, n = ws_query(kind, p, dp.DP_BF16, *args)
    assert st == dp.DP_OK and n == expect


def test_unsupported_shapes():
    assert ws_query("gn", dp.Patch(1, 8, 8, 30, 2, 0), dp.DP_BF16, 3)[0] == dp.DP_ERR_UNSUPPORTED
    assert ws_query("gn", dp.Patch(1, 8, 8, 32, 2, 0), dp.DP_BF16, 5)[0] == dp.DP_ERR_ARG
    # one thread per 16-byte channel vector, at most 1024 a block: C <= 8192 bf16, 4096 f32
    assert ws_query("gn", dp.Patch(1, 8, 8, 8192, 2, 0), dp.DP_BF16, 32)[0] == dp.DP_OK
    assert ws_query("gn", dp.Patch(1, 8, 8, 8200, 2, 0), dp.DP_BF16, 8)[0] == dp.DP_ERR_UNSUPPORTED
    assert ws_query("gn", dp.Patch(1, 8, 8, 4096, 2, 0), dp.DP_F32, 32)[0] == dp.DP_OK
    assert ws_query("gn", dp.Patch(1, 8, 8, 8192, 2, 0), dp.DP_F32, 32)[0] == dp.DP_ERR_UNSUPPORTED
    # the batch is a grid dimension (at most 65535)
    assert ws_query("gn", dp.Patch(65535, 2, 2, 8, 2, 0), dp.DP_BF16, 8)[0] == dp.DP_OK
    assert ws_query("gn", dp.Patch(65536, 2, 2, 8, 2, 0), dp.DP_BF16, 8)[0] == dp.DP_ERR_UNSUPPORTED
    # attention indexes tokens with 32-bit integers; the bf16 conv its output pixels
    assert ws_query("attn", dp.Patch(1, 1 << 16, 1 << 15, 4, 2, 0), dp.DP_F32, 1, 4)[0] == dp.DP_ERR_UNSUPPORTED
    assert ws_query("conv", dp.Patch(16384, 2048, 128, 64, 2, 0), dp.DP_BF16, 64)[0] == dp.DP_ERR_UNSUPPORTED
    assert ws_query("conv", dp.Patch(1, 8, 8, 32, 2, 0), dp.DP_BF16, 64)[0] == dp.DP_ERR_UNSUPPORTED
    assert ws_query("attn", dp.Patch(1, 8, 8, 256, 2, 0), dp.DP_BF16, 2, 128)[0] == dp.DP_ERR_UNSUPPORTED
    assert ws_query("attn", dp.Patch(1, 8, 8, 64, 2, 0), dp.DP_BF16, 2, 64)[0] == dp.DP_ERR_ARG
    assert ws_query("attn", dp.Patch(1, 8, 8, 24, 2, 0), dp.DP_F32, 1, 24)[0] == dp.DP_ERR_UNSUPPORTED


def test_groupnorm_group_count_bound():
    """The normalising block holds a thread per group: G beyond what 1024 threads (and 64 KB
    of LDS) hold is rejected on the host, with nothing enqueued."""
    # C = G = 2048 bf16: 256 channel vectors, 2048 groups -> a block of 2048 threads
    assert ws_query("gn", dp.Patch(1, 8, 8, 2048, 2, 0), dp.DP_BF16, 2048)[0] == dp.DP_ERR_UNSUPPORTED
    assert "1024" in dp.lib().dp_last_error().decode()
    assert ws_query("gn", dp.Patch(1, 8, 8, 8192, 2, 0), dp.DP_BF16, 8192)[0] == dp.DP_ERR_UNSUPPORTED
    L = dp.lib()
    p = dp._cpatch(dp.Patch(1, 8, 8, 2048, 2, 0))
    assert L.dp_groupnorm_async(p, dp.DP_BF16, 2048, 1e-5, 1, 0, FAKE, None, None, None, FAKE2, FAKE2 * 2,
                                FAKE2 * 4, 1 << 24, None) == dp.DP_ERR_UNSUPPORTED
    # the largest group counts that fit are accepted
    assert ws_query("gn", dp.Patch(1, 8, 8, 1024, 2, 0), dp.DP_BF16, 1024)[0] == dp.DP_OK
    assert ws_query("gn", dp.Patch(1, 8, 8, 2048, 2, 0), dp.DP_BF16, 1024)[0] == dp.DP_OK


def test_groupnorm_argument_errors():
    L = dp.lib()
    p = dp._cpatch(dp.Patch(1, 8, 8, 64, 2, 0))
    # eps must be positive
    assert L.dp_groupnorm_async(p, dp.DP_BF16, 8, 0.0, 0, 0, FAKE, FAKE2, None, None, None, FAKE2 * 2,
                                FAKE2 * 4, 1 << 20, None) == dp.DP_ERR_ARG
    # corrected mode needs the stale table when normalising
    assert L.dp_groupnorm_async(p, dp.DP_BF16, 8, 1e-5, 0, 0, FAKE, None, None, None, None, FAKE2 * 2,
                                FAKE2 * 4, 1 << 20, None) == dp.DP_ERR_ARG
    assert "stale_stats" in L.dp_last_error().decode()
    # workspace too small
    assert L.dp_groupnorm_async(p, dp.DP_BF16, 8, 1e-5, 0, 0, FAKE, FAKE2, None, None, None, FAKE2 * 2,
                                FAKE2 * 4, 16, None) == dp.DP_ERR_ARG
    assert "workspace" in L.dp_last_error().decode()
    # nothing requested
    assert L.dp_groupnorm_async(p, dp.DP_BF16, 8, 1e-5, 1, 0, FAKE, None, None, None, None, None,
                                FAKE2 * 4, 1 << 20, None) == dp.DP_ERR_ARG
    # unknown mode / activation
    assert L.dp_groupnorm_async(p, dp.DP_BF16, 8, 1e-5, 9, 0, FAKE, FAKE2, None, None, None, FAKE2 * 2,
                                FAKE2 * 4, 1 << 20, None) == dp.DP_ERR_ARG
    assert L.dp_groupnorm_async(p, dp.DP_BF16, 8, 1e-5, 0, 5, FAKE, FAKE2, None, None, None, FAKE2 * 2,
                                FAKE2 * 4, 1 << 20, None) == dp.DP_ERR_ARG


def test_conv_and_attention_overlap_errors():
    L = dp.lib()
    p = dp._cpatch(dp.Patch(1, 8, 8, 64, 2, 0))
    # output overlaps the stale map
    assert L.dp_conv3x3_halo(p, dp.DP_BF16, 64, FAKE, FAKE2, FAKE2 * 2, None, FAKE2 + 64, FAKE2 * 4,
                             1 << 24, None) == dp.DP_ERR_ARG
    assert "overlap" in L.dp_last_error().decode()
    pa = dp._cpatch(dp.Patch(1, 8, 8, 64, 2, 0))
    assert L.dp_attention_splice(pa, dp.DP_BF16, 1, 64, 0.0, FAKE, FAKE, FAKE, FAKE2, FAKE2, FAKE,
                                 FAKE2 * 4, 1 << 24, None) == dp.DP_ERR_ARG
    assert L.dp_attention_splice(pa, dp.DP_BF16, 1, 64, float("nan"), FAKE, FAKE, FAKE, FAKE2, FAKE2,
                                 FAKE2 * 2, FAKE2 * 4, 1 << 24, None) == dp.DP_ERR_ARG


def test_conv_rejects_images_beyond_32bit_offsets():
    # a bf16 image of 2^31 elements (16384 x 2048 x 64) cannot be addressed with 32-bit offsets
    big = dp.Patch(1, 16384, 2048, 64, 2, 0)
    assert ws_query("conv", big, dp.DP_BF16, 64)[0] == dp.DP_ERR_UNSUPPORTED
    assert "2^31" in dp.lib().dp_last_error().decode()
    assert ws_query("conv", dp.Patch(1, 16384, 2047, 64, 2, 0), dp.DP_BF16, 64)[0] == dp.DP_OK
    # the f32 direct path has no such limit
    assert ws_query("conv", big, dp.DP_F32, 64)[0] == dp.DP_OK


def test_packed_conv_weights_rejects():
    L = dp.lib()
    assert L.dp_conv3x3_packed_weights_bytes(320, 640) == 9 * 320 * 640 * 2
    assert L.dp_conv3x3_packed_weights_bytes(0, 640) == 0
    # bf16 only; Cin % 64, Cout % 32; pointers; overlap
    assert L.dp_conv3x3_pack_weights(dp.DP_F32, 64, 64, FAKE, FAKE2, None) == dp.DP_ERR_UNSUPPORTED
    assert L.dp_conv3x3_pack_weights(dp.DP_BF16, 96, 64, FAKE, FAKE2, None) == dp.DP_ERR_UNSUPPORTED
    assert L.dp_conv3x3_pack_weights(dp.DP_BF16, 64, 48, FAKE, FAKE2, None) == dp.DP_ERR_UNSUPPORTED
    assert L.dp_conv3x3_pack_weights(dp.DP_BF16, 0, 64, FAKE, FAKE2, None) == dp.DP_ERR_ARG
    assert L.dp_conv3x3_pack_weights(dp.DP_BF16, 64, 64, None, FAKE2, None) == dp.DP_ERR_ARG
    assert L.dp_conv3x3_pack_weights(dp.DP_BF16, 64, 64, FAKE, None, None) == dp.DP_ERR_ARG
    assert L.dp_conv3x3_pack_weights(dp.DP_BF16, 64, 64, FAKE, FAKE + 64, None) == dp.DP_ERR_ARG
    assert "overlap" in L.dp_last_error().decode()
    # the packed conv validates like the plain one, and is bf16 only
    p = dp._cpatch(dp.Patch(1, 8, 8, 64, 2, 0))
    assert L.dp_conv3x3_halo_packed(p, dp.DP_F32, 64, FAKE, FAKE2, FAKE2 * 2, None, FAKE2 * 3, FAKE2 * 4,
                                    1 << 24, None) == dp.DP_ERR_UNSUPPORTED
    assert L.dp_conv3x3_halo_packed(p, dp.DP_BF16, 64, FAKE, FAKE2, FAKE2 * 2, None, FAKE2 + 64, FAKE2 * 4,
                                    1 << 24, None) == dp.DP_ERR_ARG
    assert "overlap" in L.dp_last_error().decode()
    assert L.dp_conv3x3_halo_packed(p, dp.DP_BF16, 64, FAKE, FAKE2, None, None, FAKE2 * 3, FAKE2 * 4,
                                    1 << 24, None) == dp.DP_ERR_ARG
    assert "w_packed" in L.dp_last_error().decode()


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    s = torch.zeros(1, 8, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        dp.dp_stale_update(dp.Patch(1, 8, 8, 64, 4, 1), x, s)


def call_linear(dtype=dp.DP_BF16, M=16, N=64, K=64, x=FAKE, ldx=64, w=FAKE2, bias=None, y=0x30000000, ldy=64):
    return dp.lib().dp_linear(dtype, M, N, K, x, ldx, w, bias, y, ldy, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(K=48, ldx=48), dp.DP_ERR_UNSUPPORTED, "K % 64"),
    (dict(N=60, ldy=60), dp.DP_ERR_UNSUPPORTED, "multiples of 8"),
    (dict(ldx=32), dp.DP_ERR_ARG, "row strides"),
    (dict(N=0), dp.DP_ERR_ARG, "N >= 1"),
    (dict(x=0), dp.DP_ERR_ARG, "NULL"),
    (dict(y=FAKE + 8), dp.DP_ERR_ARG, "aligned"),
    (dict(y=FAKE + 512), dp.DP_ERR_ARG, "overlaps"),
    (dict(dtype=7), dp.DP_ERR_ARG, "dtype"),
])
def test_linear_rejects(kw, code, msg):
    assert call_linear(**kw) == code
    assert msg in dp.lib().dp_last_error().decode()


def test_residual_entry_points_validate():
    L = dp.lib()
    p = dp._cpatch(dp.Patch(1, 8, 8, 64, 2, 0))
    # residual overlapping the output; misaligned residual; bad layout flag
    assert L.dp_conv3x3_halo_residual(p, dp.DP_BF16, 64, FAKE, FAKE2, FAKE2 * 2, 0, None, FAKE2 * 3 + 64,
                                      FAKE2 * 3, FAKE2 * 4, 1 << 24, None) == dp.DP_ERR_ARG
    assert "overlap" in L.dp_last_error().decode()
    assert L.dp_conv3x3_halo_residual(p, dp.DP_BF16, 64, FAKE, FAKE2, FAKE2 * 2, 0, None, FAKE2 * 3 + 8,
                                      0x7000000, FAKE2 * 4, 1 << 24, None) == dp.DP_ERR_ARG
    assert "aligned" in L.dp_last_error().decode()
    assert L.dp_conv3x3_halo_residual(p, dp.DP_BF16, 64, FAKE, FAKE2, FAKE2 * 2, 2, None, None,
                                      FAKE2 * 3, FAKE2 * 4, 1 << 24, None) == dp.DP_ERR_ARG
    assert L.dp_conv3x3_halo_residual(p, dp.DP_F32, 64, FAKE, FAKE2, FAKE2 * 2, 1, None, None,
                                      FAKE2 * 3, FAKE2 * 4, 1 << 24, None) == dp.DP_ERR_UNSUPPORTED
    lin = L.dp_linear_residual
    # residual stride shorter than a row; residual overlapping y; bf16 residual stride not a multiple of 8
    assert lin(dp.DP_BF16, 16, 64, 64, FAKE, 64, FAKE2, None, 0x40000000, 32, 0x30000000, 64, None) == dp.DP_ERR_ARG
    assert lin(dp.DP_BF16, 16, 64, 64, FAKE, 64, FAKE2, None, 0x30000000 + 256, 64, 0x30000000, 64,
               None) == dp.DP_ERR_ARG
    assert "overlap" in L.dp_last_error().decode()
    assert lin(dp.DP_BF16, 16, 64, 64, FAKE, 64, FAKE2, None, 0x40000000, 68, 0x30000000, 64,
               None) == dp.DP_ERR_UNSUPPORTED


def gn_conv_ws(p, dtype, G, cout):
    out = ctypes.c_size_t(123)
    st = dp.lib().dp_groupnorm_conv3x3_halo_ws(dp._cpatch(p), dtype, G, cout, ctypes.byref(out))
    return st, out.value


@pytest.mark.parametrize("p,G,cout,fused", [
    # 256x160-tile conv, GroupNorm lanes x groups <= 512 and its parameter table in the LDS
    (dp.Patch(2, 208, 232, 128, 4, 1), 32, 192, True),
    (dp.Patch(2, 480, 480, 320, 8, 3), 32, 320, True),
    # 256x160 tiles, but C = 1664 channels' scale and shift do not fit next to the ring
    (dp.Patch(2, 128, 768, 1664, 2, 0), 32, 32, False),
    # small map (64x80 tiles, K split) and the fp32 conv: three kernels
    (dp.Patch(2, 64, 64, 320, 4, 1), 32, 320, False),
    (dp.Patch(2, 8, 6, 16, 2, 1), 4, 12, False),
])
def test_groupnorm_conv_workspace_layout(p, G, cout, fused):
    """The fused path needs only the statistics partials; otherwise a batched call normalises
    into a band in the workspace (256-byte aligned), followed by one region the GroupNorm
    partials and then the conv's split-K partials use in turn."""
    dtype = dp.DP_F32 if p.C == 16 else dp.DP_BF16
    st, n = gn_conv_ws(p, dtype, G, cout)
    assert st == dp.DP_OK
    gn = ws_query("gn", p, dtype, G)[1]
    conv = ws_query("conv", p, dtype, cout)[1]
    if fused:
        assert n == gn
    else:
        band = p.B * (p.H // p.P) * p.W * p.C * (2 if dtype == dp.DP_BF16 else 4)
        assert n == (band + 255) // 256 * 256 + max(gn, conv)
    p1 = dp.Patch(1, *list(p)[1:])
    st, n1 = gn_conv_ws(p1, dtype, G, cout)
    assert st == dp.DP_OK and n1 == max(ws_query("gn", p1, dtype, G)[1], ws_query("conv", p1, dtype, cout)[1])


def call_gn_conv(p=dp.Patch(1, 16, 32, 64, 2, 1), dtype=dp.DP_BF16, G=8, mode=0, act=1, x=FAKE,
                 table=0x50000000, fresh=None, u=FAKE2, cout=64, w=0x30000000, packed=0, res=None,
                 y=0x40000000, ws=0x60000000, ws_bytes=1 << 24):
    return dp.lib().dp_groupnorm_conv3x3_halo(dp._cpatch(p), dtype, G, 1e-5, mode, act, x, table, None, None,
                                              fresh, u, cout, w, packed, None, res, y, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code,msg", [
    ({"x": FAKE2 + 8 * 32 * 64 * 2}, dp.DP_ERR_ARG, "u_stale overlaps"),     # x_patch = band i of u_stale
    ({"y": FAKE2 + 64}, dp.DP_ERR_ARG, "y_patch overlaps"),
    ({"res": 0x40000000 + 32}, dp.DP_ERR_ARG, "y_patch overlaps"),
    ({"fresh": FAKE2}, dp.DP_ERR_ARG, "fresh_stats_out overlaps"),
    ({"fresh": 0x50000000, "mode": 2}, dp.DP_ERR_ARG, "fresh_stats_out overlaps"),   # slot 0, STALE mode
    ({"ws": FAKE2 + 1024}, dp.DP_ERR_ARG, "overlaps"),
    ({"ws_bytes": 0}, dp.DP_ERR_ARG, "workspace too small"),
    ({"y": 0}, dp.DP_ERR_ARG, "y_patch is NULL"),
    ({"u": 0}, dp.DP_ERR_ARG, "u_stale is NULL"),
    ({"table": 0}, dp.DP_ERR_ARG, "stale_stats is NULL"),
    ({"packed": 2}, dp.DP_ERR_ARG, "w_packed"),
    ({"packed": 1, "dtype": dp.DP_F32}, dp.DP_ERR_UNSUPPORTED, "bf16 only"),
    ({"cout": 48}, dp.DP_ERR_UNSUPPORTED, "Cout % 32"),
    ({"G": 7}, dp.DP_ERR_ARG, "divisible"),
    ({"mode": 5}, dp.DP_ERR_ARG, "mode"),
    ({"act": 3}, dp.DP_ERR_ARG, "activation"),
])
def test_groupnorm_conv_rejects(kw, code, msg):
    """Invalid calls fail on the host, before anything is enqueued."""
    assert call_gn_conv(**kw) == code
    assert msg in dp.lib().dp_last_error().decode()


def test_groupnorm_conv_accepts_fresh_moments_in_slot_i():
    """CORRECTED mode never reads slot i of the table, so the fresh moments may go there; the
    other checks pass too (an invalid workspace size then shows the call got that far)."""
    p = dp.Patch(1, 16, 32, 64, 2, 1)
    slot_i = 0x50000000 + 1 * 1 * 8 * 2 * 4
    assert call_gn_conv(p=p, fresh=slot_i, ws_bytes=0) == dp.DP_ERR_ARG
    assert "workspace too small" in dp.lib().dp_last_error().decode()


def call_qkv(dtype=dp.DP_BF16, M=16, N=64, K=64, x=FAKE, ldx=64, w3=FAKE2, bias3=None, yq=0x30000000, ldq=64,
             yk=0x31000000, ldk=64, yv=0x32000000, ldv=64):
    return dp.lib().dp_linear_qkv(dtype, M, N, K, x, ldx, w3, bias3, yq, ldq, yk, ldk, yv, ldv, None)


@pytest.mark.parametrize("kw,code,msg", [
    ({"yk": 0x30000000 + 64}, dp.DP_ERR_ARG, "yq overlaps yk"),
    ({"yv": FAKE2 + 128}, dp.DP_ERR_ARG, "yv overlaps an input"),
    ({"ldk": 32}, dp.DP_ERR_ARG, "row stride of yk"),
    ({"ldx": 32}, dp.DP_ERR_ARG, "ldx"),
    ({"K": 96, "ldx": 96}, dp.DP_ERR_UNSUPPORTED, "K % 64"),
    ({"ldv": 68}, dp.DP_ERR_UNSUPPORTED, "multiples of 8"),
    ({"yq": 0}, dp.DP_ERR_ARG, "yq is NULL"),
    ({"yk": 0x31000000 + 8}, dp.DP_ERR_ARG, "aligned"),
    ({"N": 0}, dp.DP_ERR_ARG, "N >= 1"),
    ({"dtype": 9}, dp.DP_ERR_ARG, "dtype"),
])
def test_linear_qkv_rejects(kw, code, msg):
    assert call_qkv(**kw) == code
    assert msg in dp.lib().dp_last_error().decode()


def test_linear_qkv_empty_is_noop():
    assert call_qkv(M=0, x=0, yq=0, yk=0, yv=0) == dp.DP_OK
