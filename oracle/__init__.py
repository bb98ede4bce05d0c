"""CPU oracle of the displaced-patch layer (DistriFusion), float64, numpy.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain reference that the
GPU library is checked against.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the library never does, and the
oracle imports nothing from the library.  Every function computes from its
inputs in float64 with no intermediate rounding.

``displaced``: one patch's share of a layer step against stale state
               (GroupNorm corrected/local/stale, conv with stale halo rows,
               attention over spliced K/V, band splice).
``sync``:      the synchronous full-image layer used for warm-up steps and to
               build the stale state of a displaced step.

Parity pins: each function is checked in the CPU test suite against
torch.nn.functional (group_norm, conv2d, scaled_dot_product_attention in
float64), brute-force loops on tiny maps, and the invariants the method fixes
(stale == fresh gives the synchronous layer, one patch gives the plain layer).
"""

from .displaced import (GN_CORRECTED, GN_LOCAL, GN_STALE, attention_proj_splice, attention_splice, band,
                        conv3x3_halo, displaced_layer, displaced_step_all, gn_async, gn_band_stats,
                        gn_moments, linear, silu, splice, splice_tokens, stale_update)
from .sync import attention, band_moments, conv3x3, group_norm, project, self_attention, sync_layer

__all__ = [
    "GN_CORRECTED", "GN_LOCAL", "GN_STALE", "attention_proj_splice", "attention_splice", "linear",
    "attention", "project", "band", "conv3x3_halo",
    "displaced_layer", "displaced_step_all", "gn_async", "gn_band_stats", "gn_moments", "silu", "splice",
    "splice_tokens", "stale_update", "band_moments", "conv3x3", "group_norm",
    "self_attention", "sync_layer",
]
