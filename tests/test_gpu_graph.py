"""A displaced layer step captured as a HIP graph: every replay equals the eager step bit for bit.

The step's calls only launch kernels on the current stream (no allocation, no
host synchronisation, no memset), so the step can be captured once and
replayed; bench.py times the step that way.  Between replays the test runs
eager work of its own (torch kernels, a synchronisation) and overwrites every
output, so each replay has to recompute everything.
"""

import pytest
import torch

from displaced_patch_parallelism_amd import synth
from displaced_patch_parallelism_amd.configs import CONFIGS
from displaced_patch_parallelism_amd.layers import DisplacedLayer
from tests.gpu_util import announce

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


@pytest.mark.parametrize("name", ["c0", "c1", "c3", "c2p", "c1r", "c2t"])
def test_graph_replays_match_eager(name):
    announce("graph replay", name)
    c = CONFIGS[name]
    inp = synth.layer_inputs(c, 0)
    dev = torch.device("cuda:0")
    layer = DisplacedLayer(c, inp.convs, dev, projs=inp.projs)
    to = lambda a: torch.from_numpy(a).to(dev, layer.dt).contiguous()  # noqa: E731
    layer.warmup(to(inp.x_prev))
    i = c.patch
    xb = to(inp.x[:, i * c.h:(i + 1) * c.h])
    outs = [o for _, _, done in layer.calls(xb, i) for o in done]
    layer.step(xb, i)
    torch.cuda.synchronize()
    eager = [bits(o).clone() for o in outs]
    eager_tables = {k: t.clone() for k, t in layer.tables.items()}

    graph = layer.capture(xb, i)
    for r in range(3):
        junk = torch.randn(1 << 20, device=dev)
        _ = (junk * junk).sum().item()               # eager work and a synchronisation
        for o in outs:
            o.fill_(float(r + 7))
        for t in layer.tables.values():
            t[i].fill_(-1.0)
        graph.replay()
        torch.cuda.synchronize()
        for k, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(bits(o), e), f"{name} replay {r} output {k}"
        for k, t in layer.tables.items():
            assert torch.equal(t, eager_tables[k]), f"{name} replay {r} statistics table {k}"
