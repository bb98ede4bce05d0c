"""The seeded input generator: rounding, determinism, distributions (CPU only)."""

import numpy as np
import torch

from displaced_patch_parallelism_amd import synth
from displaced_patch_parallelism_amd.configs import CONFIGS


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -1.00390625, 3.0e-39, 65504.0], np.float32)])
    ours = synth.bf16_round(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    assert ours.tobytes() == ref.tobytes()


def test_same_seed_same_inputs():
    cfg = CONFIGS["c0"]
    a, b = synth.layer_inputs(cfg, 7), synth.layer_inputs(cfg, 7)
    assert a.x.tobytes() == b.x.tobytes() and a.x_prev.tobytes() == b.x_prev.tobytes()
    assert a.convs[0][0].tobytes() == b.convs[0][0].tobytes()
    c = synth.layer_inputs(cfg, 8)
    assert a.x.tobytes() != c.x.tobytes()


def test_distributions():
    cfg = CONFIGS["c1"]
    inp = synth.layer_inputs(cfg, 0)
    assert inp.x.shape == (1, 128, 128, 320)
    assert abs(inp.x.mean()) < 0.01 and abs(inp.x.std() - 1) < 0.01
    d = inp.x_prev - inp.x
    assert abs(d.std() - 0.05) < 0.002
    w, b = inp.convs[0]
    assert w.shape == (320, 3, 3, 320) and b.dtype == np.float32
    assert abs(w.std() * np.sqrt(9 * 320) - 1) < 0.02
    assert synth.bf16_round(w).tobytes() == w.tobytes()


def test_trajectory_is_a_small_random_walk():
    from displaced_patch_parallelism_amd.configs import LayerConfig
    cfg = LayerConfig("t", "f32", B=1, H=16, W=16, C=32, G=8, P=2, graph=("gn_silu", "conv"))
    tr = synth.trajectory(cfg, seed=3, steps=4)
    assert len(tr.xs) == 5 and len(tr.convs) == 1
    rng = np.random.default_rng(3)
    x0 = rng.standard_normal((1, 16, 16, 32), dtype=np.float32)
    np.testing.assert_array_equal(tr.xs[0], x0)
    for a, b in zip(tr.xs[:-1], tr.xs[1:]):
        d = (b - a).ravel()
        assert abs(d.std() - 0.05) < 0.005 and abs(d.mean()) < 0.005
    again = synth.trajectory(cfg, seed=3, steps=4)
    for a, b in zip(tr.xs, again.xs):
        np.testing.assert_array_equal(a, b)
