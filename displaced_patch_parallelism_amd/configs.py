"""Layer shapes of the displaced-patch workloads (pure data, no arithmetic).

Each entry is one UNet-layer shape on which one patch's share of a denoising
step is computed.  The maps are split into ``P`` equal row bands; patch ``i``
owns rows ``[i*H/P, (i+1)*H/P)``.  The graph is the order of the layer's
steps:

* ``gn``       corrected asynchronous GroupNorm
* ``gn_silu``  the same, followed by SiLU
* ``conv``     3x3 convolution whose halo rows come from the stale map
* ``attn``     self-attention, queries from the fresh patch, keys/values from
               the stale map with the fresh patch spliced in
* ``attn_proj`` the same with learned Q/K/V/O projections (the stale context is
               the previous step's projected K/V cache)
* ``conv_res`` / ``attn_proj_res``  the conv / projected attention with the
               layer's own input added to the output (the skip connection of a
               ResNet or transformer block of the U-Net)

Shapes follow the SDXL-like levels the method is applied to (DistriFusion
summary on atlas.scime.ai, "Experimental setup"; the 1024px and 3840px
resolutions of "Key results").
"""

from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class LayerConfig:
    name: str
    dtype: str            # "f32" or "bf16": storage type of activations and weights
    B: int
    H: int
    W: int
    C: int
    G: int                # GroupNorm groups
    P: int                # patches (row bands)
    graph: Tuple[str, ...]
    heads: int = 0        # attention heads (0: no attention in the graph)
    head_dim: int = 0
    eps: float = 1e-5
    patch: int = 1        # the patch index a benchmark step computes
    steps: int = 1        # denoising steps the layer test runs (1 warm-up + displaced)
    note: str = ""

    @property
    def h(self) -> int:
        return self.H // self.P

    @property
    def N(self) -> int:
        return self.H * self.W

    @property
    def Nq(self) -> int:
        return self.h * self.W

    @property
    def n_conv(self) -> int:
        return sum(s in ("conv", "conv_res") for s in self.graph)

    @property
    def n_proj(self) -> int:
        return sum(s in ("attn_proj", "attn_proj_res") for s in self.graph)

    @property
    def n_attn(self) -> int:
        return sum(s == "attn" for s in self.graph) + self.n_proj

    @property
    def has_attn(self) -> bool:
        return self.n_attn > 0

    @property
    def has_proj(self) -> bool:
        return self.n_proj > 0

    @property
    def has_conv(self) -> bool:
        return self.n_conv > 0

    def conv_flops(self) -> float:
        """Multiply-adds x2 of the patch's 3x3 convs (Cout = Cin = C), all of them."""
        return self.n_conv * 2.0 * self.B * self.Nq * self.C * 9 * self.C

    def attn_flops(self) -> float:
        """QK^T plus PV, 2 flops per multiply-add, every (query, key) pair, every attention."""
        return self.n_attn * 4.0 * self.B * self.heads * self.Nq * self.N * self.head_dim

    def proj_flops(self) -> float:
        """The four C x C projections (Q, K, V, O) of the patch's tokens, every projected attention."""
        return self.n_proj * 4 * 2.0 * self.B * self.Nq * self.C * self.C

    def band_bytes(self) -> int:
        """Bytes of one activation band [B][h][W][C]."""
        return self.B * self.Nq * self.C * (4 if self.dtype == "f32" else 2)


CONFIGS = {
    "c0": LayerConfig(
        "c0", "f32", B=1, H=16, W=16, C=32, G=8, P=2,
        graph=("gn_silu", "conv", "attn"), heads=1, head_dim=32, steps=2,
        note="tiny block: GN+SiLU, conv3x3 32->32, 1-head attention over 256 tokens"),
    "c1": LayerConfig(
        "c1", "bf16", B=1, H=128, W=128, C=320, G=32, P=4,
        graph=("gn_silu", "conv"),
        note="SDXL level-1 conv layer at 1024px: GN+SiLU, conv3x3 320->320"),
    "c2": LayerConfig(
        "c2", "bf16", B=1, H=64, W=64, C=640, G=32, P=4,
        graph=("gn", "attn", "conv"), heads=10, head_dim=64,
        note="SDXL level-2 attention layer: GN, 10x64 attention over 4096 tokens, conv3x3 640->640"),
    "c3": LayerConfig(
        "c3", "bf16", B=1, H=32, W=32, C=1280, G=32, P=8,
        graph=("gn", "attn", "conv"), heads=20, head_dim=64,
        note="SDXL level-3 attention layer: GN, 20x64 attention over 1024 tokens, conv3x3 1280->1280"),
    "c4a": LayerConfig(
        "c4a", "bf16", B=1, H=480, W=480, C=320, G=32, P=8,
        graph=("gn_silu", "conv"),
        note="3840px conv layer: GN+SiLU, conv3x3 320->320, 60x480 bands"),
    "c4b": LayerConfig(
        "c4b", "bf16", B=1, H=240, W=240, C=640, G=32, P=8,
        graph=("gn", "attn"), heads=10, head_dim=64,
        note="3840px attention layer: GN, 10x64 attention, 7200 queries over 57600 keys"),
    # The two attention layers again with learned Q/K/V/O projections: the stale context is
    # the previous step's projected K and V maps.
    "c2p": LayerConfig(
        "c2p", "bf16", B=1, H=64, W=64, C=640, G=32, P=4,
        graph=("gn", "attn_proj", "conv"), heads=10, head_dim=64,
        note="c2 with Q/K/V/O projections 640->640 and a projected K/V cache"),
    "c4bp": LayerConfig(
        "c4bp", "bf16", B=1, H=240, W=240, C=640, G=32, P=8,
        graph=("gn", "attn_proj"), heads=10, head_dim=64,
        note="c4b with Q/K/V/O projections 640->640 and a projected K/V cache"),
    # SDXL-like blocks of the U-Net: a ResNet block (two GroupNorm+SiLU -> conv pairs, the
    # second conv adding the block input) and a transformer block's attention (GroupNorm,
    # Q/K/V projections, attention over the projected K/V cache, output projection adding
    # the block input)
    "c1r": LayerConfig(
        "c1r", "bf16", B=1, H=128, W=128, C=320, G=32, P=4,
        graph=("gn_silu", "conv", "gn_silu", "conv_res"),
        note="SDXL level-1 ResNet block at 1024px: (GN+SiLU, conv3x3 320->320) x 2, skip added"),
    "c2t": LayerConfig(
        "c2t", "bf16", B=1, H=64, W=64, C=640, G=32, P=4,
        graph=("gn", "attn_proj_res"), heads=10, head_dim=64,
        note="SDXL level-2 transformer-block attention: GN, Q/K/V 640->640, 10x64 attention, "
             "O projection with the block input added"),
}

# Workloads made of several layers, each a patch step of its own (the one-GPU share of one
# denoising step at that resolution touches every layer once).
COMPOSITES = {
    "c4": ("c4a", "c4b"),
}
