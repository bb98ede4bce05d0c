"""dp_stale_update on the GPU: bit-exact band splice, canaries, statistics table."""

import numpy as np
import pytest
import torch

import displaced_patch_parallelism_amd as dp
from displaced_patch_parallelism_amd.configs import CONFIGS
from tests.gpu_util import announce, dev

pytestmark = pytest.mark.gpu


def bits(t):
    return t.detach().cpu().view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


@pytest.mark.parametrize("name", list(CONFIGS))
def test_band_splice_bit_exact_every_patch(name):
    c = CONFIGS[name]
    dt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    g = torch.Generator(device="cpu").manual_seed(1)
    stale = torch.randn((c.B, c.H, c.W, c.C), generator=g).to(dt).to(dev())
    for i in ([0, 1, c.P - 1] if c.P > 2 else range(c.P)):
        announce("splice", name, "patch", i)
        before = bits(stale)
        patch = torch.randn((c.B, c.h, c.W, c.C), generator=g).to(dt).to(dev())
        dp.dp_stale_update(dp.Patch(c.B, c.H, c.W, c.C, c.P, i), patch, stale)
        torch.cuda.synchronize()
        after = bits(stale)
        r0, r1 = i * c.h, (i + 1) * c.h
        assert np.array_equal(after[:, r0:r1], bits(patch))
        assert np.array_equal(after[:, :r0], before[:, :r0])
        assert np.array_equal(after[:, r1:], before[:, r1:])


@pytest.mark.parametrize("B,H,W,C,P,dt", [(2, 6, 5, 3, 3, torch.float32), (3, 4, 7, 5, 2, torch.bfloat16),
                                          (2, 8, 4, 16, 4, torch.bfloat16), (1, 9, 3, 1, 3, torch.float32)])
def test_ragged_and_batched(B, H, W, C, P, dt):
    """Spans that are not 16-byte multiples, and B > 1 (one span per batch)."""
    announce("splice ragged", B, H, W, C, P, dt)
    g = torch.Generator(device="cpu").manual_seed(2)
    stale = torch.randn((B, H, W, C), generator=g).to(dt).to(dev())
    h = H // P
    for i in range(P):
        ref = stale.clone()
        patch = torch.randn((B, h, W, C), generator=g).to(dt).to(dev())
        dp.dp_stale_update(dp.Patch(B, H, W, C, P, i), patch, stale)
        ref[:, i * h:(i + 1) * h] = patch
        assert np.array_equal(bits(stale), bits(ref))


def test_in_place_band_is_noop_and_stats_table():
    announce("splice in-place + stats table")
    stale = torch.randn((1, 8, 4, 8), device=dev()).to(torch.bfloat16)
    before = bits(stale)
    dp.dp_stale_update(dp.Patch(1, 8, 4, 8, 4, 2), stale[:, 4:6], stale)
    torch.cuda.synchronize()
    assert np.array_equal(bits(stale), before)
    table = torch.randn((4, 1, 8, 2), device=dev())
    fresh = torch.randn((1, 8, 2), device=dev())
    ref = table.clone()
    ref[2] = fresh
    dp.dp_stats_update(4, 2, fresh, table)
    assert torch.equal(table, ref)
