"""Seeded synthetic inputs, shared by the tests, the benchmark and the smoke check.

This module holds none of the displaced-patch arithmetic.  It only draws
random numbers, rounds inputs to the storage type, and forms the previous
step's input ``x' = x + 0.05 * eps`` that defines the workload (consecutive
diffusion steps see nearly identical inputs: DistriFusion abstract on
scholarfeed.org; "input temporal redundancy" in the PipeFusion explainer on
gist.science, Problem Statement).

Conventions
-----------
* Generator: ``numpy.random.default_rng(seed)`` (PCG64), drawing in float32.
* Draw order for a layer: fresh map ``x``, perturbation ``eps``, then for each
  conv of the graph (``conv`` or ``conv_res``) its weights and its bias, then
  for each projected attention step (``attn_proj`` or ``attn_proj_res``) its
  Q, K, V and O weights and biases (N(0, 1/C)).
* Weights ``[Cout][3][3][Cin]`` and bias ``[Cout]`` are N(0, 1/fan_in) with
  fan_in = 9*Cin.  The bias stays float32; weights are rounded to the
  activation storage type.
* bf16 rounding is round-to-nearest-even on the float32 bit pattern; the
  returned arrays are float32 holding exactly representable bf16 values, so
  every consumer reads identical numbers.
"""

from dataclasses import dataclass
from typing import List, Optional, Tuple

import numpy as np

PERTURB = 0.05
CONV_STEPS = ("conv", "conv_res")               # graph steps that own a conv's weights
PROJ_STEPS = ("attn_proj", "attn_proj_res")     # graph steps that own Q/K/V/O projections


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.asarray(a, dtype=np.float32)
    if dtype == "bf16":
        return bf16_round(a)
    if dtype == "f32":
        return np.ascontiguousarray(a)
    raise ValueError(f"unknown dtype {dtype!r}")


def conv_params(rng: np.random.Generator, cin: int, cout: int,
                dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    std = np.float32(1.0 / np.sqrt(9.0 * cin))
    w = rng.standard_normal((cout, 3, 3, cin), dtype=np.float32) * std
    b = rng.standard_normal((cout,), dtype=np.float32) * std
    return to_storage(w, dtype), b.astype(np.float32)


def map_pair(rng: np.random.Generator, shape, dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """A fresh map ~ N(0,1) and its stale version fresh + 0.05*N(0,1)."""
    fresh = rng.standard_normal(shape, dtype=np.float32)
    eps = rng.standard_normal(shape, dtype=np.float32)
    stale = fresh + np.float32(PERTURB) * eps
    return to_storage(fresh, dtype), to_storage(stale, dtype)


def proj_params(rng: np.random.Generator, C: int, dtype: str) -> Tuple[np.ndarray, ...]:
    """(wq, bq, wk, bk, wv, bv, wo, bo): weights [C][C] and biases [C], N(0, 1/C)."""
    std = np.float32(1.0 / np.sqrt(C))
    out = []
    for _ in range(4):
        w = rng.standard_normal((C, C), dtype=np.float32) * std
        b = rng.standard_normal((C,), dtype=np.float32) * std
        out += [to_storage(w, dtype), b.astype(np.float32)]
    return tuple(out)


@dataclass
class LayerInputs:
    """Raw inputs of one layer: current-step input, previous-step input, weights."""
    x: np.ndarray            # [B][H][W][C] fresh (current step) layer input
    x_prev: np.ndarray       # [B][H][W][C] previous step's layer input
    convs: List[Tuple[np.ndarray, np.ndarray]]
    projs: List[Tuple[np.ndarray, ...]] = None   # per attn_proj step: (wq, bq, wk, bk, wv, bv, wo, bo)


def layer_inputs(cfg, seed: int, perturb: float = PERTURB) -> LayerInputs:
    """Inputs of a whole layer per the config: x, eps, then each conv's w and b."""
    rng = np.random.default_rng(seed)
    shape = (cfg.B, cfg.H, cfg.W, cfg.C)
    x = rng.standard_normal(shape, dtype=np.float32)
    eps = rng.standard_normal(shape, dtype=np.float32)
    x_prev = x + np.float32(perturb) * eps
    convs = [conv_params(rng, cfg.C, cfg.C, cfg.dtype)
             for s in cfg.graph if s in CONV_STEPS]
    projs = [proj_params(rng, cfg.C, cfg.dtype) for s in cfg.graph if s in PROJ_STEPS]
    return LayerInputs(to_storage(x, cfg.dtype), to_storage(x_prev, cfg.dtype), convs, projs)


@dataclass
class Trajectory:
    """Inputs of one layer over several denoising steps (see ``trajectory``)."""
    xs: List[np.ndarray]     # steps + 1 maps [B][H][W][C]: xs[0] feeds the warm-up step
    convs: List[Tuple[np.ndarray, np.ndarray]]
    projs: List[Tuple[np.ndarray, ...]] = None


def trajectory(cfg, seed: int, steps: int, perturb: float = PERTURB) -> Trajectory:
    """A slowly drifting layer input: x_0 ~ N(0,1), x_t = x_{t-1} + 0.05*N(0,1).

    Draw order: x_0, then each step's perturbation, then each conv's w and b.
    Accumulated in float32 and rounded to the storage type per step.
    """
    rng = np.random.default_rng(seed)
    shape = (cfg.B, cfg.H, cfg.W, cfg.C)
    x = rng.standard_normal(shape, dtype=np.float32)
    xs = [to_storage(x, cfg.dtype)]
    for _ in range(steps):
        x = x + np.float32(perturb) * rng.standard_normal(shape, dtype=np.float32)
        xs.append(to_storage(x, cfg.dtype))
    convs = [conv_params(rng, cfg.C, cfg.C, cfg.dtype) for s in cfg.graph if s in CONV_STEPS]
    projs = [proj_params(rng, cfg.C, cfg.dtype) for s in cfg.graph if s in PROJ_STEPS]
    return Trajectory(xs, convs, projs)


@dataclass
class ConvCase:
    fresh: np.ndarray      # [B][H][W][Cin] current map (its band i is the patch)
    stale: np.ndarray      # [B][H][W][Cin] previous step's map
    w: np.ndarray          # [Cout][3][3][Cin]
    bias: np.ndarray       # [Cout] float32


def conv_case(B, H, W, cin, cout, dtype, seed) -> ConvCase:
    rng = np.random.default_rng(seed)
    fresh, stale = map_pair(rng, (B, H, W, cin), dtype)
    w, b = conv_params(rng, cin, cout, dtype)
    return ConvCase(fresh, stale, w, b)


@dataclass
class AttnCase:
    q: np.ndarray          # [B][N][C] current queries (band i is the patch)
    k: np.ndarray          # [B][N][C] current keys
    v: np.ndarray          # [B][N][C] current values
    k_stale: np.ndarray    # [B][N][C] previous step's keys
    v_stale: np.ndarray    # [B][N][C] previous step's values


def attn_case(B, N, C, dtype, seed, q_scale: float = 1.0) -> AttnCase:
    """Independent Q, K, V maps (so operand mix-ups show) and stale K, V."""
    rng = np.random.default_rng(seed)
    q = to_storage(rng.standard_normal((B, N, C), dtype=np.float32) * np.float32(q_scale), dtype)
    k, k_stale = map_pair(rng, (B, N, C), dtype)
    v, v_stale = map_pair(rng, (B, N, C), dtype)
    return AttnCase(q, k, v, k_stale, v_stale)


def gn_case(B, H, W, C, dtype, seed, mean: float = 0.0,
            affine: bool = False) -> Tuple[np.ndarray, np.ndarray, Optional[np.ndarray], Optional[np.ndarray]]:
    """A fresh map, its stale version, and optional GroupNorm affine parameters."""
    rng = np.random.default_rng(seed)
    fresh, stale = map_pair(rng, (B, H, W, C), dtype)
    if mean:
        fresh = to_storage(fresh + np.float32(mean), dtype)
        stale = to_storage(stale + np.float32(mean), dtype)
    gamma = beta = None
    if affine:
        gamma = (1.0 + 0.5 * rng.standard_normal((C,), dtype=np.float32)).astype(np.float32)
        beta = (0.5 * rng.standard_normal((C,), dtype=np.float32)).astype(np.float32)
    return fresh, stale, gamma, beta
