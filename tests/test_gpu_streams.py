"""Calls on two streams at once, each with the binding's default workspace, give the results
the same calls give one after another (the default scratch is per stream)."""

import pytest
import torch

import displaced_patch_parallelism_amd as dp
from displaced_patch_parallelism_amd import synth
from displaced_patch_parallelism_amd.configs import CONFIGS
from tests.gpu_util import announce, gpu

pytestmark = pytest.mark.gpu


def test_default_workspace_is_per_stream():
    c = CONFIGS["c3"]          # conv split along K over 8 workgroups: both calls use scratch
    announce("two streams, default workspaces, c3 GroupNorm + conv")
    p = dp.Patch(1, c.H, c.W, c.C, c.P, c.patch)
    cases = []
    for seed in (11, 12):
        case = synth.conv_case(1, c.H, c.W, c.C, c.C, "bf16", seed)
        xb = gpu(case.fresh[:, c.patch * c.h:(c.patch + 1) * c.h], "bf16")
        cases.append((xb, gpu(case.stale, "bf16"), gpu(case.w, "bf16"), gpu(case.bias, "f32")))
    table = torch.rand((c.P, 1, c.G, 2), device="cuda") + 0.5

    def run(xb, stale, w, bias):
        y, st = dp.dp_groupnorm_async(p, xb, c.G, table)
        return y, st, dp.dp_conv3x3_halo(p, y, stale, w, bias)

    refs = [run(*cs) for cs in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = [[], []]
    for _ in range(8):
        for k, s in enumerate(streams):
            with torch.cuda.stream(s):
                outs[k].append(run(*cases[k]))
    torch.cuda.synchronize()
    for k in range(2):
        for got in outs[k]:
            for g, r in zip(got, refs[k]):
                assert torch.equal(g.view(torch.int16) if g.dtype == torch.bfloat16 else g,
                                   r.view(torch.int16) if r.dtype == torch.bfloat16 else r)
