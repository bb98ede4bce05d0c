"""dp_attention_splice on the GPU against the oracle, per call, on identical inputs."""

import numpy as np
import pytest
import torch

import displaced_patch_parallelism_amd as dp
import oracle
from displaced_patch_parallelism_amd import synth
from displaced_patch_parallelism_amd.configs import CONFIGS
from tests.gpu_util import announce, assert_parity, gpu, host

pytestmark = pytest.mark.gpu


def run_case(B, H, W, heads, d, P, i, dtype, seed=0, rows=None, q_scale=1.0):
    C = heads * d
    case = synth.attn_case(B, H * W, C, dtype, seed, q_scale=q_scale)
    nq = (H // P) * W
    t0 = i * nq
    q, k, v = (a[:, t0:t0 + nq] for a in (case.q, case.k, case.v))
    ref = oracle.attention_splice(q, k, v, case.k_stale, case.v_stale, H, W, P, i, heads, rows=rows)
    o = dp.dp_attention_splice(dp.Patch(B, H, W, C, P, i), heads, gpu(q, dtype), gpu(k, dtype), gpu(v, dtype),
                               gpu(case.k_stale, dtype), gpu(case.v_stale, dtype))
    torch.cuda.synchronize()
    got = host(o)
    if rows is not None:
        got = got[:, rows]
    assert_parity(got, ref, dtype, f"attn {dtype} B{B} {H}x{W} {heads}x{d} P{P} i{i}")
    return o


@pytest.mark.parametrize("name", ["c0", "c2", "c3"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_config_shapes(name, seed):
    c = CONFIGS[name]
    patches = [0, c.patch, c.P - 1] if c.P > 2 else list(range(c.P))
    for i in patches:
        announce("attention", name, "patch", i, "seed", seed)
        run_case(c.B, c.H, c.W, c.heads, c.head_dim, c.P, i, c.dtype, seed=20 + 10 * seed + i)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_c4b_sampled_rows(seed):
    """3840px layer: the oracle computes a seeded sample of query rows plus every band-edge row."""
    c = CONFIGS["c4b"]
    rng = np.random.default_rng(seed)
    nq = c.Nq
    edges = list(range(c.W)) + list(range(nq - c.W, nq))
    rows = sorted(set(rng.choice(nq, 256, replace=False).tolist()) | set(edges))
    announce("attention c4b sampled", len(rows), "rows", "seed", seed)
    run_case(c.B, c.H, c.W, c.heads, c.head_dim, c.P, c.patch, c.dtype, seed=5 + seed, rows=rows)


@pytest.mark.parametrize("B,H,W,heads,P,i", [
    (1, 5, 13, 2, 5, 2),     # N = 65: ragged last key tile; Nq = 13
    (2, 6, 30, 3, 3, 1),     # batch 2, Nq = 60, N = 180, band straddles key tiles
    (1, 40, 10, 1, 2, 1),    # Nq = 200: ragged query tile
    (1, 8, 24, 4, 1, 0),     # one patch: plain self-attention
    (2, 48, 90, 1, 2, 1),    # Nq = 2160 (8-wave tiles, ragged), N = 4320 (ragged key tiles), batch 2
    (1, 4, 8, 1, 2, 1),      # N = 32: the whole map is one partial key tile
    (1, 48, 32, 1, 8, 3),    # one query tile over 24 key tiles: 12 key splits of 2 tiles, merged
])
def test_ragged_bf16(B, H, W, heads, P, i):
    announce("attention ragged", B, H, W, heads, P, i)
    run_case(B, H, W, heads, 64, P, i, "bf16", seed=i)


@pytest.mark.parametrize("B,H,W,heads,P,i", [
    (1, 4, 8, 1, 2, 1),      # N = 32: one ragged key tile
    (1, 8, 8, 1, 2, 0),      # N = 64: one full tile
    (1, 4, 24, 2, 2, 1),     # 2 tiles, the last ragged
    (1, 6, 32, 1, 2, 1),     # 3 tiles
    (1, 8, 32, 1, 2, 0),     # 4 tiles: one whole pass of the loop unrolled by the ring depth
    (1, 8, 40, 1, 4, 3),     # 5 tiles
    (1, 12, 32, 1, 3, 1),    # 6 tiles
    (1, 10, 44, 1, 2, 1),    # 7 tiles, the last with 56 keys
    (2, 10, 48, 1, 2, 1),    # 8 tiles, the last ragged, batch 2
    (1, 9, 64, 2, 3, 2),     # 9 tiles
    (1, 12, 48, 3, 4, 2),    # 9 tiles in 4 key splits of 2, 2, 2 and 3
])
def test_key_tile_counts_bf16(B, H, W, heads, P, i):
    """Every count of 64-key tiles per key split from 1 to 9, full and ragged: the tile loop's
    prologue, its pipelined iterations and the unrolled loop's partial last pass."""
    announce("attention tile counts", B, H, W, heads, P, i)
    run_case(B, H, W, heads, 64, P, i, "bf16", seed=50 + H + W)


@pytest.mark.parametrize("q_scale", [4.0, 8.0, 16.0])
def test_peaked_softmax_bf16(q_scale):
    """Large scores (queries scaled x4, x8, x16: score standard deviations of about 4, 8 and 16,
    so a few keys dominate each softmax) exercise the running-offset rescaling and the precision
    of the scaled scores."""
    announce("attention peaked", q_scale)
    run_case(1, 16, 32, 2, 64, 4, 2, "bf16", seed=9, q_scale=q_scale)
    run_case(1, 64, 64, 10, 64, 4, 1, "bf16", seed=10, q_scale=q_scale)


@pytest.mark.parametrize("order", ["rising", "falling"])
@pytest.mark.parametrize("i", [1, 3])
def test_score_steps_move_offset(order, i):
    """Scores that step by about 11.5 (in units of log2 of the softmax weight) every 24 keys: rising,
    every step is a new maximum more than 2^8 above the kernel's running offset, so the check on
    each 32-key half's probability sum fails and the offset moves, in first and second halves of
    tiles alike (steps at keys 24, 48, 72, ... fall in both) and in every key split; falling, the
    first tile holds the maximum and the offset never moves.  A missed rescale would weight an
    earlier level 2^11 times too much."""
    B, H, W, heads, d, P = 1, 64, 64, 2, 64, 4
    C, N = heads * d, H * W
    rng = np.random.default_rng(31 + i)
    a = rng.choice([-1.0, 1.0], size=(heads, d)).astype(np.float32)      # one direction per head
    lvl = (np.arange(N) // 24).astype(np.float32)
    if order == "falling":
        lvl = lvl[::-1].copy()
    scale = 1.0 / np.sqrt(d)
    # q ~ a, k_n = lvl_n a (integers, exact in bf16): scale * log2(e) * q.k_n ~ 11.5 * lvl_n
    k_full = synth.to_storage((lvl[:, None, None] * a[None]).reshape(B, N, C), "bf16")
    q_full = synth.to_storage((a[None] + 0.05 * rng.standard_normal((N, heads, d))).reshape(B, N, C), "bf16")
    v_full = synth.to_storage(rng.standard_normal((B, N, C)), "bf16")
    y = scale * np.log2(np.e) * np.einsum("hd,nhd->nh", a, k_full.reshape(N, heads, d).astype(np.float64))
    if order == "rising":
        assert np.min(np.diff(y[24::24, 0])) > 8.0        # every step exceeds the lazy margin
    nq = (H // P) * W
    t0 = i * nq
    q, k, v = (x[:, t0:t0 + nq] for x in (q_full, k_full, v_full))
    announce("attention score steps", order, "patch", i)
    ref = oracle.attention_splice(q, k, v, k_full, v_full, H, W, P, i, heads)
    o = dp.dp_attention_splice(dp.Patch(B, H, W, C, P, i), heads, gpu(q, "bf16"), gpu(k, "bf16"), gpu(v, "bf16"),
                               gpu(k_full, "bf16"), gpu(v_full, "bf16"))
    torch.cuda.synchronize()
    assert_parity(host(o), ref, "bf16", f"attn score steps {order} i{i}")


@pytest.mark.parametrize("d", [4, 16, 32, 64, 128])
def test_f32_head_dims(d):
    announce("attention f32 d", d)
    run_case(1, 8, 8, 2, d, 2, 1, "f32", seed=d)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 32)])
def test_onehot_splice_indexing_bit_exact(dtype, d):
    """Each query selects one key by a margin of 1000 (every other softmax weight is
    exactly 0); the output row is then that key's V row: fresh (negative values)
    inside the band, stale (positive) outside."""
    N = 2 * d                                  # keys n = +-e_{n mod d}: all distinct
    W, P = 16, 4
    H = N // W
    nq = (H // P) * W
    rng = np.random.default_rng(3)
    sign = np.where(np.arange(N) < d, 1.0, -1.0).astype(np.float32)
    kdir = np.zeros((N, d), np.float32)
    kdir[np.arange(N), np.arange(N) % d] = sign
    v_fresh = -rng.integers(1, 101, size=(1, N, d)).astype(np.float32)
    v_stale = rng.integers(1, 101, size=(1, N, d)).astype(np.float32)
    k = kdir[None]
    for i in range(P):
        announce("attention one-hot", dtype, d, "patch", i)
        t0 = i * nq
        targets = rng.integers(0, N, size=nq)
        q = 1000.0 * kdir[targets][None]
        ref = oracle.attention_splice(q, k[:, t0:t0 + nq], v_fresh[:, t0:t0 + nq], k, v_stale, H, W, P, i, 1,
                                      scale=1.0)
        inband = ((targets >= t0) & (targets < t0 + nq))[None, :, None]
        assert np.array_equal(ref, np.where(inband, v_fresh[:, targets], v_stale[:, targets]))
        o = dp.dp_attention_splice(dp.Patch(1, H, W, d, P, i), 1, gpu(q, dtype), gpu(k[:, t0:t0 + nq], dtype),
                                   gpu(v_fresh[:, t0:t0 + nq], dtype), gpu(k, dtype), gpu(v_stale, dtype),
                                   scale=1.0)
        assert np.array_equal(host(o), ref), f"patch {i}"


def test_in_place_splice_alias_and_determinism():
    """k_patch/v_patch pointing into band i of the stale maps gives the same result."""
    c = CONFIGS["c2"]
    announce("attention alias c2")
    case = synth.attn_case(1, c.N, c.C, "bf16", 4)
    i, nq = 1, c.Nq
    p = dp.Patch(1, c.H, c.W, c.C, c.P, i)
    q = gpu(case.q[:, i * nq:(i + 1) * nq], "bf16")
    k = gpu(case.k[:, i * nq:(i + 1) * nq], "bf16")
    v = gpu(case.v[:, i * nq:(i + 1) * nq], "bf16")
    ks, vs = gpu(case.k_stale, "bf16"), gpu(case.v_stale, "bf16")
    o1 = dp.dp_attention_splice(p, c.heads, q, k, v, ks, vs)
    o2 = dp.dp_attention_splice(p, c.heads, q, k, v, ks, vs)
    ks2, vs2 = ks.clone(), vs.clone()
    ks2[:, i * nq:(i + 1) * nq] = k
    vs2[:, i * nq:(i + 1) * nq] = v
    o3 = dp.dp_attention_splice(p, c.heads, q, ks2[:, i * nq:(i + 1) * nq], vs2[:, i * nq:(i + 1) * nq], ks2, vs2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
