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
