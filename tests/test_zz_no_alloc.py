"""dp_groupnorm_async_noalloc (statistics partials in the library's static scratch) against
dp_groupnorm_async (caller workspace), through the C ABI, on the GPU.

Two calls in a row, the second on a smaller input, each checked bit for bit against the
workspace entry point on the same inputs (same kernels, same plan), and the first also against
the oracle; a call whose partials exceed the scratch is rejected on the host.
"""

import ctypes

import numpy as np
import pytest
import torch

import displaced_patch_parallelism_amd as dp
import oracle
from displaced_patch_parallelism_amd import synth
from tests.gpu_util import announce, assert_parity, gpu, host

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 1 << 20


def ws_bytes(p, dtype, G):
    out = ctypes.c_size_t(0)
    assert dp.lib().dp_groupnorm_async_ws(dp._cpatch(p), dtype, G, ctypes.byref(out)) == dp.DP_OK
    return out.value


def run_pair(B, H, W, C, G, P, i, dtype, mode, act, seed):
    """Both entry points on the same inputs; returns (noalloc outputs, workspace outputs, inputs)."""
    fresh, stale, gamma, beta = synth.gn_case(B, H, W, C, dtype, seed, affine=True)
    table = oracle.band_moments(stale, G, P).astype(np.float32)
    h = H // P
    xb = fresh[:, i * h:(i + 1) * h]
    p = dp.Patch(B, H, W, C, P, i)
    code = dp.DP_BF16 if dtype == "bf16" else dp.DP_F32
    need = ws_bytes(p, code, G)
    assert 0 < need <= SCRATCH_BYTES
    x, tab, ga, be = gpu(xb, dtype), gpu(table, "f32"), gpu(gamma, "f32"), gpu(beta, "f32")
    outs = []
    L = dp.lib()
    stream = torch.cuda.current_stream().cuda_stream
    mode_c, act_c = dp.GN_MODES[mode], dp.ACTS[act]
    for noalloc in (True, False):
        y = torch.full_like(x, 3.0)
        st = torch.full((B, G, 2), -1.0, dtype=torch.float32, device=x.device)
        if noalloc:
            rc = L.dp_groupnorm_async_noalloc(dp._cpatch(p), code, G, 1e-5, mode_c, act_c, x.data_ptr(),
                                              tab.data_ptr(), ga.data_ptr(), be.data_ptr(), st.data_ptr(),
                                              y.data_ptr(), stream)
        else:
            ws = torch.empty(need, dtype=torch.uint8, device=x.device)
            rc = L.dp_groupnorm_async(dp._cpatch(p), code, G, 1e-5, mode_c, act_c, x.data_ptr(), tab.data_ptr(),
                                      ga.data_ptr(), be.data_ptr(), st.data_ptr(), y.data_ptr(), ws.data_ptr(),
                                      need, stream)
        assert rc == dp.DP_OK, L.dp_last_error().decode()
        outs.append((y, st))
    torch.cuda.synchronize()
    return outs, (xb, table, gamma, beta)


def test_noalloc_matches_workspace_entry_point_twice():
    # first call: the c1 band (228 statistics blocks); second: a smaller, ragged band
    cases = [(1, 128, 128, 320, 32, 4, 1, "bf16", "corrected", "silu", 1),
             (1, 12, 10, 48, 6, 3, 2, "bf16", "stale", None, 2)]
    for n, (B, H, W, C, G, P, i, dtype, mode, act, seed) in enumerate(cases):
        announce("groupnorm noalloc call", n, (B, H, W, C, G, P, i), dtype, mode, act)
        outs, (xb, table, gamma, beta) = run_pair(B, H, W, C, G, P, i, dtype, mode, act, seed)
        (yn, sn), (yw, sw) = outs
        assert torch.equal(yn.view(torch.int16), yw.view(torch.int16)), f"call {n}: y differs"
        assert torch.equal(sn, sw), f"call {n}: fresh moments differ"
        if n == 0:
            ref_y, ref_st = oracle.gn_async(xb, table, P, i, G, 1e-5, oracle.GN_CORRECTED, gamma, beta, act)
            assert_parity(host(yn), ref_y, dtype, "noalloc y vs oracle")
            np.testing.assert_allclose(host(sn), ref_st, rtol=1e-4, atol=1e-5)


def test_noalloc_rejects_partials_beyond_the_scratch():
    p = dp.Patch(32, 64, 64, 320, 4, 1)
    assert ws_bytes(p, dp.DP_BF16, 32) > SCRATCH_BYTES
    L = dp.lib()
    rc = L.dp_groupnorm_async_noalloc(dp._cpatch(p), dp.DP_BF16, 32, 1e-5, 0, 0, 0x10000, 0x20000, None, None,
                                      0x30000, 0x40000, None)
    assert rc == dp.DP_ERR_UNSUPPORTED
    assert "scratch" in L.dp_last_error().decode()
