"""Independent float64 references built from torch.nn.functional on the CPU.

They pin the oracle: each is the textbook operation applied to the map a
patch sees (the previous step's map with the fresh band spliced in), written
with torch's library routines rather than the oracle's numpy code.
"""

import numpy as np
import torch
import torch.nn.functional as F


def t64(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float64))


def spliced_map(stale, fresh_band, r0):
    """stale map [B][H][W][C] with rows r0.. replaced by the band (torch indexing)."""
    m = t64(stale).clone()
    band = t64(fresh_band)
    m[:, r0:r0 + band.shape[1]] = band
    return m


def nhwc_to_nchw(t):
    return t.permute(0, 3, 1, 2).contiguous()


def nchw_to_nhwc(t):
    return t.permute(0, 2, 3, 1).contiguous()


def group_norm_nhwc(x, G, eps=1e-5, gamma=None, beta=None):
    x = t64(x)
    y = F.group_norm(nhwc_to_nchw(x), G,
                     None if gamma is None else t64(gamma),
                     None if beta is None else t64(beta), eps)
    return nchw_to_nhwc(y)


def conv2d_nhwc(x, w, bias):
    """w [Cout][3][3][Cin] -> torch [Cout][Cin][3][3]."""
    wt = t64(w).permute(0, 3, 1, 2).contiguous()
    y = F.conv2d(nhwc_to_nchw(t64(x)), wt, None if bias is None else t64(bias), padding=1)
    return nchw_to_nhwc(y)


def sdpa_tokens(q, k, v, heads, scale=None):
    """q [B][Nq][C], k/v [B][N][C] -> [B][Nq][C] via scaled_dot_product_attention."""
    q, k, v = t64(q), t64(k), t64(v)
    B, Nq, C = q.shape
    d = C // heads

    def split(t):
        return t.reshape(B, t.shape[1], heads, d).permute(0, 2, 1, 3).contiguous()

    o = F.scaled_dot_product_attention(split(q), split(k), split(v), scale=scale)
    return o.permute(0, 2, 1, 3).reshape(B, Nq, C)
