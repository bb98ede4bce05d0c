"""dp_linear (the learned projections) on the GPU against the oracle's linear."""

import numpy as np
import pytest
import torch

import displaced_patch_parallelism_amd as dp
import oracle
from displaced_patch_parallelism_amd import synth
from tests.gpu_util import announce, assert_parity, gpu, host

pytestmark = pytest.mark.gpu


def case(M, N, K, dtype, seed):
    rng = np.random.default_rng(seed)
    x = synth.to_storage(rng.standard_normal((M, K), dtype=np.float32), dtype)
    w = synth.to_storage(rng.standard_normal((N, K), dtype=np.float32) / np.float32(np.sqrt(K)), dtype)
    b = rng.standard_normal((N,), dtype=np.float32)
    return x, w, b


@pytest.mark.parametrize("M,N,K", [
    (1024, 640, 640),     # c2p projections (64x64 tiles)
    (7200, 640, 640),     # c4bp projections (128x128 tiles)
    (100, 136, 128),      # ragged rows and columns
    (1, 8, 64),
    (130, 1280, 1280),    # c3-sized width
])
def test_bf16_shapes(M, N, K):
    announce("linear", M, N, K)
    x, w, b = case(M, N, K, "bf16", M + N)
    y = dp.dp_linear(gpu(x, "bf16"), gpu(w, "bf16"), gpu(b, "f32"))
    torch.cuda.synchronize()
    assert_parity(host(y), oracle.linear(x, w, b), "bf16", f"linear {M}x{N}x{K}")


def test_bf16_strided_rows_into_a_band_and_no_bias():
    """x rows strided inside a wider buffer, y written into band rows of a token map."""
    M, N, K = 96, 64, 128
    x, w, _ = case(M, N, K, "bf16", 5)
    big = torch.zeros((M, K + 64), dtype=torch.bfloat16, device="cuda")
    big[:, 32:32 + K] = gpu(x, "bf16")
    tokens = torch.full((4 * M, N), 7.0, dtype=torch.bfloat16, device="cuda")   # 4 bands of M rows
    band = tokens[M:2 * M]
    dp.dp_linear(big[:, 32:32 + K], gpu(w, "bf16"), None, y=band)
    torch.cuda.synchronize()
    assert_parity(host(band), oracle.linear(x, w), "bf16", "linear strided")
    t = host(tokens)
    assert np.all(t[:M] == 7.0) and np.all(t[2 * M:] == 7.0)


def test_empty_and_f32():
    x, w, b = case(0, 64, 64, "bf16", 1)
    y = dp.dp_linear(gpu(np.zeros((0, 64), np.float32), "bf16"), gpu(w, "bf16"), gpu(b, "f32"))
    assert y.shape == (0, 64)
    for M, N, K in [(5, 3, 7), (33, 40, 16)]:
        x, w, b = case(M, N, K, "f32", 2)
        y = dp.dp_linear(gpu(x, "f32"), gpu(w, "f32"), gpu(b, "f32"))
        torch.cuda.synchronize()
        assert_parity(host(y), oracle.linear(x, w, b), "f32", f"linear f32 {M}x{N}x{K}")


def test_deterministic():
    x, w, b = case(1024, 640, 640, "bf16", 9)
    xs, ws, bs = gpu(x, "bf16"), gpu(w, "bf16"), gpu(b, "f32")
    y1 = dp.dp_linear(xs, ws, bs)
    y2 = dp.dp_linear(xs, ws, bs)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("M,N,K,dtype", [
    (1024, 640, 640, "bf16"),    # c2t output projection (64x64 tiles)
    (7200, 640, 640, "bf16"),    # 128x128 tiles
    (100, 136, 128, "bf16"),     # ragged rows and columns
    (33, 40, 16, "f32"),
])
def test_residual(M, N, K, dtype):
    """The skip connection is added before rounding: y = x W^T + b + r."""
    announce("linear residual", M, N, K, dtype)
    x, w, b = case(M, N, K, dtype, M + 3)
    r = synth.to_storage(np.random.default_rng(M).standard_normal((M, N), dtype=np.float32), dtype)
    y = dp.dp_linear_residual(gpu(x, dtype), gpu(w, dtype), gpu(b, "f32"), gpu(r, dtype))
    torch.cuda.synchronize()
    assert_parity(host(y), oracle.linear(x, w, b) + r, dtype, f"linear residual {M}x{N}x{K}")
    # no residual: exactly dp_linear
    y0 = dp.dp_linear_residual(gpu(x, dtype), gpu(w, dtype), gpu(b, "f32"), None)
    y1 = dp.dp_linear(gpu(x, dtype), gpu(w, dtype), gpu(b, "f32"))
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


def test_residual_strided_rows():
    """Residual rows strided inside a wider buffer (a band of a token map)."""
    M, N, K = 96, 64, 128
    x, w, b = case(M, N, K, "bf16", 6)
    r = synth.to_storage(np.random.default_rng(8).standard_normal((M, N), dtype=np.float32), "bf16")
    big = torch.zeros((M, N + 64), dtype=torch.bfloat16, device="cuda")
    big[:, 16:16 + N] = gpu(r, "bf16")
    y = dp.dp_linear_residual(gpu(x, "bf16"), gpu(w, "bf16"), gpu(b, "f32"), big[:, 16:16 + N])
    torch.cuda.synchronize()
    assert_parity(host(y), oracle.linear(x, w, b) + r, "bf16", "linear residual strided")


@pytest.mark.parametrize("M,N,K,dtype", [
    (1024, 640, 640, "bf16"),    # c2p's Q/K/V: one [1024][1920] product on 64x64 tiles
    (7200, 640, 640, "bf16"),    # c4bp's: 128x128 tiles
    (100, 96, 128, "bf16"),      # ragged rows; 64-column tiles straddle the segment edges
    (1, 8, 64, "bf16"),
    (33, 40, 16, "f32"),
])
def test_qkv_equals_three_linears(M, N, K, dtype):
    """dp_linear_qkv gives bit for bit the three dp_linear outputs (and the oracle's values)."""
    announce("linear qkv", M, N, K, dtype)
    rng = np.random.default_rng(M + 2 * N)
    x = synth.to_storage(rng.standard_normal((M, K), dtype=np.float32), dtype)
    ws = [synth.to_storage(rng.standard_normal((N, K), dtype=np.float32) / np.float32(np.sqrt(K)), dtype)
          for _ in range(3)]
    bs = [rng.standard_normal((N,), dtype=np.float32) for _ in range(3)]
    xg = gpu(x, dtype)
    w3 = gpu(np.concatenate(ws), dtype)
    b3 = gpu(np.concatenate(bs), "f32")
    outs = dp.dp_linear_qkv(xg, w3, b3)
    refs = [dp.dp_linear(xg, gpu(w, dtype), gpu(b, "f32")) for w, b in zip(ws, bs)]
    torch.cuda.synchronize()
    for s, (o, r) in enumerate(zip(outs, refs)):
        bits = (lambda t: t.view(torch.int16)) if dtype == "bf16" else (lambda t: t.view(torch.int32))
        assert torch.equal(bits(o), bits(r)), f"segment {s}"
        assert_parity(host(o), oracle.linear(x, ws[s], bs[s]), dtype, f"qkv segment {s}")


def test_qkv_into_strided_bands_without_bias():
    """Q into a scratch buffer, K and V straight into band rows of two token maps (row stride
    wider than N), no bias; rows outside the bands are untouched."""
    M, N, K = 96, 64, 128
    rng = np.random.default_rng(21)
    x = synth.to_storage(rng.standard_normal((M, K), dtype=np.float32), "bf16")
    w3 = synth.to_storage(rng.standard_normal((3 * N, K), dtype=np.float32) / np.float32(np.sqrt(K)), "bf16")
    kmap = torch.full((4 * M, N + 32), 5.0, dtype=torch.bfloat16, device="cuda")
    vmap = torch.full((4 * M, N + 32), 6.0, dtype=torch.bfloat16, device="cuda")
    q, k, v = dp.dp_linear_qkv(gpu(x, "bf16"), gpu(w3, "bf16"), None, yk=kmap[2 * M:3 * M, :N],
                               yv=vmap[M:2 * M, 16:16 + N])
    torch.cuda.synchronize()
    for s, got in enumerate((q, k, v)):
        assert_parity(host(got), oracle.linear(x, w3[s * N:(s + 1) * N]), "bf16", f"qkv strided {s}")
    km, vm = host(kmap), host(vmap)
    assert np.all(km[:2 * M] == 5.0) and np.all(km[3 * M:] == 5.0) and np.all(km[2 * M:3 * M, N:] == 5.0)
    assert np.all(vm[:M] == 6.0) and np.all(vm[2 * M:] == 6.0) and np.all(vm[M:2 * M, :16] == 6.0)
    assert np.all(vm[M:2 * M, 16 + N:] == 6.0)
