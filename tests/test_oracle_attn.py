"""Pins of the oracle's attention over spliced K/V (CPU only).

DistriFusion keeps the full spatial K and V of every layer on every device
(PipeFusion explainer on gist.science, Problem Statement and Memory
Efficiency); the patch's queries attend to all of them, its own band being
fresh.  Pins: torch scaled_dot_product_attention with spliced K/V, brute
force on tiny inputs, closed forms (one key; identical keys) and an exact
one-hot case that names the buffer each value row came from.
"""

import itertools
import math

import numpy as np
import pytest

import oracle
from displaced_patch_parallelism_amd import synth
from tests.torch_refs import sdpa_tokens, t64


def spliced_tokens(stale, band_tokens, t0):
    s = t64(stale).clone()
    s[:, t0:t0 + band_tokens.shape[1]] = t64(band_tokens)
    return s


@pytest.mark.parametrize("B,H,W,heads,d,P", [(1, 4, 4, 1, 8, 2), (2, 6, 5, 2, 4, 3),
                                             (1, 8, 8, 4, 16, 4), (1, 3, 7, 2, 8, 1)])
def test_matches_torch_sdpa_with_spliced_kv(B, H, W, heads, d, P):
    C = heads * d
    case = synth.attn_case(B, H * W, C, "f32", seed=H * W * C)
    h = H // P
    for i in range(P):
        t0, t1 = i * h * W, (i + 1) * h * W
        q, k, v = case.q[:, t0:t1], case.k[:, t0:t1], case.v[:, t0:t1]
        out = oracle.attention_splice(q, k, v, case.k_stale, case.v_stale, H, W, P, i, heads)
        ref = sdpa_tokens(q, spliced_tokens(case.k_stale, k, t0), spliced_tokens(case.v_stale, v, t0), heads)
        np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-12)


def brute_attention(q, K, V, heads, scale):
    B, Nq, C = q.shape
    d = C // heads
    out = np.zeros((B, Nq, C))
    for b, e, n in itertools.product(range(B), range(heads), range(Nq)):
        sl = slice(e * d, (e + 1) * d)
        scores = [scale * sum(float(q[b, n, c]) * float(K[b, m, c]) for c in range(sl.start, sl.stop))
                  for m in range(K.shape[1])]
        top = max(scores)
        wts = [math.exp(s - top) for s in scores]
        tot = sum(wts)
        for c in range(sl.start, sl.stop):
            out[b, n, c] = sum(wt * float(V[b, m, c]) for m, wt in enumerate(wts)) / tot
    return out


def test_brute_force_tiny():
    H, W, heads, d, P = 4, 3, 2, 3, 2
    case = synth.attn_case(1, H * W, heads * d, "f32", seed=31)
    for i in range(P):
        t0, t1 = i * 6, (i + 1) * 6
        K = case.k_stale.copy(); K[:, t0:t1] = case.k[:, t0:t1]
        V = case.v_stale.copy(); V[:, t0:t1] = case.v[:, t0:t1]
        out = oracle.attention_splice(case.q[:, t0:t1], case.k[:, t0:t1], case.v[:, t0:t1],
                                      case.k_stale, case.v_stale, H, W, P, i, heads, scale=0.7)
        np.testing.assert_allclose(out, brute_attention(case.q[:, t0:t1], K, V, heads, 0.7),
                                   rtol=0, atol=1e-12)


def test_single_key_returns_its_value():
    case = synth.attn_case(1, 1, 8, "f32", seed=2)
    out = oracle.attention_splice(case.q, case.k, case.v, case.k_stale, case.v_stale, 1, 1, 1, 0, 2)
    np.testing.assert_array_equal(out, case.v.astype(np.float64))


def test_identical_keys_average_values():
    H, W, C = 4, 2, 4
    case = synth.attn_case(1, H * W, C, "f32", seed=3)
    k = np.ones((1, 4, C), np.float32)
    k_stale = np.ones((1, H * W, C), np.float32)
    out = oracle.attention_splice(case.q[:, :4], k, case.v[:, :4], k_stale, case.v_stale, H, W, 2, 0, 1)
    V = case.v_stale.astype(np.float64).copy(); V[:, :4] = case.v[:, :4]
    np.testing.assert_allclose(out, np.broadcast_to(V.mean(axis=1, keepdims=True), out.shape),
                               rtol=0, atol=1e-14)


def test_onehot_softmax_names_the_buffer():
    """Each query selects one key by a margin that makes the softmax exactly one-hot."""
    H, W, P, C = 4, 4, 2, 16
    N = H * W
    rng = np.random.default_rng(5)
    eye = np.eye(C, dtype=np.float32)
    k_full = eye[np.arange(N) % C][None]           # key n = e_{n mod 16}
    v_fresh = -rng.integers(1, 101, size=(1, N, C)).astype(np.float32)
    v_stale = rng.integers(1, 101, size=(1, N, C)).astype(np.float32)
    for i in range(P):
        t0, t1 = i * 8, (i + 1) * 8
        targets = rng.integers(0, N, size=t1 - t0)
        q = 1000.0 * eye[targets][None]                # scores 1000 vs 0: exp(-1000) == 0
        out = oracle.attention_splice(q, k_full[:, t0:t1], v_fresh[:, t0:t1], k_full, v_stale,
                                      H, W, P, i, 1, scale=1.0)
        for n, tgt in enumerate(targets):
            want = v_fresh[0, tgt] if t0 <= tgt < t1 else v_stale[0, tgt]
            np.testing.assert_array_equal(out[0, n], want)


def test_rows_subset_and_default_scale():
    H, W, heads, d, P = 4, 4, 2, 8, 2
    case = synth.attn_case(1, H * W, heads * d, "f32", seed=6)
    args = (case.q[:, 8:], case.k[:, 8:], case.v[:, 8:], case.k_stale, case.v_stale, H, W, P, 1, heads)
    full = oracle.attention_splice(*args)
    np.testing.assert_array_equal(oracle.attention_splice(*args, rows=[0, 5, 7]), full[:, [0, 5, 7]])
    np.testing.assert_allclose(oracle.attention_splice(*args, scale=d ** -0.5), full, rtol=0, atol=0)
