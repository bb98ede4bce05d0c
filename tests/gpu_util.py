"""Helpers for the GPU parity tests: tensors, tolerances, printing the case."""

import sys

import numpy as np
import torch

# Tolerances of the displaced-patch hot path (per call, per output tensor):
#   f32:  rel-L2 <= 1e-4
#   bf16: rel-L2 <= 2e-2 and max-abs <= 5e-2
# Splice and halo/splice indexing cases are bit-exact.
TOL = {"f32": {"rel_l2": 1e-4, "max_abs": None}, "bf16": {"rel_l2": 2e-2, "max_abs": 5e-2}}


def dev():
    return torch.device("cuda:0")


def gpu(a, dtype):
    """numpy float32 (bf16-representable when dtype is bf16) -> GPU tensor, exact."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(dev(), {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]).contiguous()


def host(t):
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    diff = got - ref
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    mab = float(np.abs(diff).max()) if diff.size else 0.0
    return rel, mab


def assert_parity(got, ref, dtype, what=""):
    rel, mab = errors(got, ref)
    tol = TOL[dtype]
    msg = f"{what}: rel-L2 {rel:.3e} (tol {tol['rel_l2']}), max-abs {mab:.3e} (tol {tol['max_abs']})"
    assert np.all(np.isfinite(np.asarray(got))), what + ": non-finite output"
    assert rel <= tol["rel_l2"], msg
    if tol["max_abs"] is not None:
        assert mab <= tol["max_abs"], msg
    return rel, mab


def announce(*parts):
    """Print (and flush) what case is about to run on the GPU."""
    print("[gpu case]", *parts, flush=True)
    sys.stdout.flush()


def assert_table(got, ref, dtype, k, what=""):
    """A GroupNorm statistics table against the oracle's.  The first GroupNorm step (k == 0)
    reads the layer input itself, identical bits on both sides, so its fp32 moments are held to
    1e-4; a later GroupNorm step normalises an intermediate the GPU stores in the layer's dtype
    (rounded) while the oracle keeps it in float64, so its moments get that dtype's tolerance."""
    if k == 0 or dtype == "f32":
        np.testing.assert_allclose(got, ref, rtol=1e-4, atol=1e-4, err_msg=what)
    else:
        assert_parity(got, ref, dtype, what)
