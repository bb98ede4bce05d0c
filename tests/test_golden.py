"""The oracle still reproduces its stored tiny-layer fixture (CPU only)."""
import json
import os

import numpy as np

from tests.golden.make_golden import build

HERE = os.path.dirname(os.path.abspath(__file__))


def test_tiny_layer_fixture():
    with open(os.path.join(HERE, "golden", "tiny_layer.json")) as f:
        stored = json.load(f)
    now = build()
    assert stored["graph"] == now["graph"]
    for a, b in zip(stored["outputs"], now["outputs"]):
        np.testing.assert_allclose(np.array(a), np.array(b), rtol=0, atol=1e-13)
