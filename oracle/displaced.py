"""Displaced-patch layer for one patch, in float64 -- the oracle's core.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources (the pages are web text about DistriFusion; no equation of the paper
is on them, so each step below is the plainest reading the pages support):

* "DistriFusion: Distributed Parallel Inference for High-Resolution Diffusion
  Models" (study.space), Method: the input image is divided into patches, one
  per device, and slightly outdated activations of the previous step
  ("activation displacement") give each patch its context.
* DistriFusion summary (atlas.scime.ai), Approach: stale activations of the
  previous denoising step are reused, the AllGather overlaps compute, and a
  corrected asynchronous GroupNorm fixes the statistics.  Same page, table
  "Measured effects reported in the paper": the GroupNorm ablations
  (on-device statistics only, stale statistics reused, synchronised exact
  statistics).
* PipeFusion explainer (gist.science), Problem Statement and Memory
  Efficiency: DistriFusion keeps the full spatial K and V of every layer on
  every device.

Readings taken where the pages are silent:

* Patches are equal row bands of an NHWC map: patch i owns rows
  [i*H/P, (i+1)*H/P); token n of a map is row n // W, column n % W.
* The map a patch "sees" is the previous step's map with its own fresh band
  spliced in (``splice``).  The conv reads it through a zero-padded 3x3
  window, so only the stale rows just above and below the band matter; the
  attention uses all of it as K and V.
* Corrected GroupNorm uses the statistics of that spliced map: the stale
  global moments with patch i's stale share replaced by its fresh share,
  applied to E[x] and E[x^2]; variance = E[x^2] - E[x]^2 clamped at 0.
"""

import numpy as np

F64 = np.float64

GN_CORRECTED = 0   # fresh local + stale others (the method)
GN_LOCAL = 1       # on-device patch statistics only (ablation)
GN_STALE = 2       # previous step's statistics only (ablation)


def band(H, P, i):
    """Rows [r0, r1) owned by patch i of P equal row bands."""
    if H % P != 0 or not (0 <= i < P):
        raise ValueError("H must be divisible by P and 0 <= i < P")
    h = H // P
    return i * h, (i + 1) * h


def splice(stale_map, patch, P, i):
    """The map as patch i sees it: stale everywhere, its fresh band in rows r0..r1."""
    full = np.array(stale_map, dtype=F64, copy=True)
    r0, r1 = band(full.shape[1], P, i)
    if patch.shape != full[:, r0:r1].shape:
        raise ValueError("patch shape does not match band")
    full[:, r0:r1] = patch
    return full


# --------------------------------------------------------------------------
# GroupNorm, corrected asynchronous form
# --------------------------------------------------------------------------

def gn_band_stats(x_patch, G):
    """Per (batch, group): (mean, mean of squares) over the band. Returns [B][G][2]."""
    x = np.asarray(x_patch, dtype=F64)
    B, C = x.shape[0], x.shape[-1]
    if C % G != 0:
        raise ValueError("C must be divisible by G")
    xg = x.reshape(B, -1, G, C // G)
    m = xg.mean(axis=(1, 3))
    q = (xg * xg).mean(axis=(1, 3))
    return np.stack([m, q], axis=-1)


def gn_moments(fresh, stale_table, P, i, mode):
    """Group moments (E[x], E[x^2]) per (batch, group) that the patch normalises with.

    fresh: [B][G][2] band statistics of the current step;
    stale_table: [P][B][G][2] per-band statistics of the previous step.
    """
    fresh = np.asarray(fresh, dtype=F64)
    if mode == GN_LOCAL:
        return fresh[..., 0], fresh[..., 1]
    stale = np.asarray(stale_table, dtype=F64)
    if stale.shape[0] != P:
        raise ValueError("stale table must hold P bands")
    if mode == GN_STALE:
        tot = stale.sum(axis=0) / P
    elif mode == GN_CORRECTED:
        others = stale.sum(axis=0) - stale[i]
        tot = (fresh + others) / P
    else:
        raise ValueError("unknown GroupNorm mode")
    return tot[..., 0], tot[..., 1]


def silu(y):
    return y / (1.0 + np.exp(-y))


def gn_async(x_patch, stale_table, P, i, G, eps=1e-5, mode=GN_CORRECTED,
             gamma=None, beta=None, act=None):
    """Normalise patch i; returns (y_patch, fresh band statistics [B][G][2])."""
    x = np.asarray(x_patch, dtype=F64)
    B, C = x.shape[0], x.shape[-1]
    fresh = gn_band_stats(x, G)
    mu, q = gn_moments(fresh, stale_table, P, i, mode)
    var = np.maximum(q - mu * mu, 0.0)
    rstd = 1.0 / np.sqrt(var + eps)
    cg = C // G
    mu_c = np.repeat(mu, cg, axis=1).reshape(B, *([1] * (x.ndim - 2)), C)
    rstd_c = np.repeat(rstd, cg, axis=1).reshape(B, *([1] * (x.ndim - 2)), C)
    y = (x - mu_c) * rstd_c
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=F64)
    if beta is not None:
        y = y + np.asarray(beta, dtype=F64)
    if act == "silu":
        y = silu(y)
    elif act not in (None, "none"):
        raise ValueError("unknown activation")
    return y, fresh


# --------------------------------------------------------------------------
# 3x3 convolution with stale halo rows
# --------------------------------------------------------------------------

def conv3x3_halo(x_patch, x_stale, w, bias, P, i):
    """3x3 cross-correlation, stride 1, zero padding, of patch i's rows of the spliced map.

    x_patch [B][h][W][Cin], x_stale [B][H][W][Cin], w [Cout][3][3][Cin], bias [Cout] or None.
    Output [B][h][W][Cout]:  out[b,y,x,o] = bias[o] + sum_{ky,kx,c} w[o,ky,kx,c] *
    src[b, r0+y+ky-1, x+kx-1, c], with src = splice(x_stale, x_patch) and zero outside.
    """
    full = splice(x_stale, x_patch, P, i)
    B, H, W, C = full.shape
    r0, r1 = band(H, P, i)
    h = r1 - r0
    w = np.asarray(w, dtype=F64)
    if w.shape[1:] != (3, 3, C):
        raise ValueError("weights must be [Cout][3][3][Cin]")
    padded = np.zeros((B, H + 2, W + 2, C), dtype=F64)
    padded[:, 1:H + 1, 1:W + 1] = full
    out = np.zeros((B, h, W, w.shape[0]), dtype=F64)
    for ky in range(3):
        for kx in range(3):
            # source row r0+y+ky-1 sits at padded row r0+y+ky
            window = padded[:, r0 + ky:r0 + ky + h, kx:kx + W, :]
            out += window @ w[:, ky, kx, :].T
    if bias is not None:
        out += np.asarray(bias, dtype=F64)
    return out


# --------------------------------------------------------------------------
# Attention over the stale K/V with the fresh patch spliced in
# --------------------------------------------------------------------------

def splice_tokens(stale_tokens, patch_tokens, H, W, P, i):
    """Token-major [B][N][C] form of ``splice``: tokens of rows r0..r1 come from the patch."""
    full = np.array(stale_tokens, dtype=F64, copy=True)
    r0, r1 = band(H, P, i)
    if full.shape[1] != H * W or patch_tokens.shape[1] != (r1 - r0) * W:
        raise ValueError("token counts do not match the map")
    full[:, r0 * W:r1 * W] = patch_tokens
    return full


def attention_splice(q_patch, k_patch, v_patch, k_stale, v_stale, H, W, P, i,
                     heads, scale=None, rows=None, chunk=512):
    """softmax(scale * Q K^T) V per head, K and V spliced.

    q_patch, k_patch, v_patch: [B][Nq][C]; k_stale, v_stale: [B][N][C] with
    N = H*W, Nq = (H/P)*W and C = heads*d.  Head e uses channels [e*d, (e+1)*d).
    ``scale`` defaults to d**-0.5.  ``rows`` optionally restricts the output to
    those query indices (the result then has len(rows) tokens).
    Returns O [B][Nq or len(rows)][C].
    """
    K = splice_tokens(k_stale, np.asarray(k_patch, F64), H, W, P, i)
    V = splice_tokens(v_stale, np.asarray(v_patch, F64), H, W, P, i)
    Q = np.asarray(q_patch, dtype=F64)
    if rows is not None:
        Q = Q[:, np.asarray(rows)]
    B, Nq, C = Q.shape
    if C % heads != 0:
        raise ValueError("C must be heads * head_dim")
    d = C // heads
    if scale is None or scale <= 0:
        scale = d ** -0.5
    out = np.empty((B, Nq, C), dtype=F64)
    for b in range(B):
        for e in range(heads):
            sl = slice(e * d, (e + 1) * d)
            Kh, Vh = K[b, :, sl], V[b, :, sl]
            for s in range(0, Nq, chunk):
                S = scale * (Q[b, s:s + chunk, sl] @ Kh.T)
                S -= S.max(axis=1, keepdims=True)
                E = np.exp(S)
                out[b, s:s + chunk, sl] = (E @ Vh) / E.sum(axis=1, keepdims=True)
    return out


# --------------------------------------------------------------------------
# Learned projections of an attention layer
# --------------------------------------------------------------------------

def linear(x, w, bias=None):
    """y = x W^T + bias over the last axis: x [..][K], w [N][K], bias [N] (or None)."""
    y = np.asarray(x, dtype=F64) @ np.asarray(w, dtype=F64).T
    if bias is not None:
        y = y + np.asarray(bias, dtype=F64)
    return y


def attention_proj_splice(h_tokens, proj, k_stale, v_stale, H, W, P, i, heads, scale=None):
    """Attention layer with learned projections for patch i.

    The fresh patch's queries, keys and values are its projections
    (Q, K, V = h W_q^T + b_q, ...); every device keeps the full K and V maps of
    the layer from the previous step (PipeFusion explainer on gist.science,
    Problem Statement and Memory Efficiency), so the stale context of the other
    bands is those cached projections, and the fresh K and V replace band i.
    The output is the attention projected by W_o.  Returns (O, K, V) with O
    [B][Nq][C] and the fresh K, V [B][Nq][C] that refresh the cache.
    """
    wq, bq, wk, bk, wv, bv, wo, bo = proj
    q = linear(h_tokens, wq, bq)
    k = linear(h_tokens, wk, bk)
    v = linear(h_tokens, wv, bv)
    a = attention_splice(q, k, v, k_stale, v_stale, H, W, P, i, heads, scale)
    return linear(a, wo, bo), k, v


# --------------------------------------------------------------------------
# Splice of the fresh band into the resident stale buffer
# --------------------------------------------------------------------------

def stale_update(stale, x_patch, P, i):
    """Copy of ``stale`` with band i replaced by the patch, bit for bit (same dtype)."""
    out = np.array(stale, copy=True)
    r0, r1 = band(out.shape[1], P, i)
    if x_patch.shape != out[:, r0:r1].shape:
        raise ValueError("patch shape does not match band")
    out[:, r0:r1] = x_patch
    return out


# --------------------------------------------------------------------------
# One displaced layer step of patch i
# --------------------------------------------------------------------------

def displaced_layer(graph, params, x_patch, state, P, i, gn_mode=GN_CORRECTED):
    """Run patch i of a layer graph against the previous step's state.

    graph: sequence of "gn", "gn_silu", "conv", "attn", "attn_proj", and the residual
           forms "conv_res" / "attn_proj_res", whose output adds the layer's own input
           patch (the skip connection of a ResNet or transformer block).
    params: dict with G, eps, heads, scale (optional), gamma/beta (optional),
            convs: list of (w, bias) in graph order, projs: list of
            (wq, bq, wk, bk, wv, bv, wo, bo) for the attn_proj steps in order.
    state: dict with "stats" {step index: [P][B][G][2] GroupNorm moments per band of
           the previous step, one table per GroupNorm step} and "maps": {step index:
           [B][H][W][C] stale input map of that conv or attention step; (step index,
           "k") / (step index, "v"): the previous step's projected K / V maps of an
           attn_proj step}.
    Returns (outputs, new_state): outputs is the list of every step's patch
    output (float64); new_state is the state with patch i's band and
    statistics spliced in.
    """
    x_in = np.asarray(x_patch, dtype=F64)
    h = x_in
    B, hb, W, C = h.shape
    H = hb * P
    outputs = []
    new_stats = {k: np.array(t, dtype=F64, copy=True) for k, t in state["stats"].items()}
    new_maps = {k: np.array(v, dtype=F64, copy=True) for k, v in state["maps"].items()}
    conv_iter = iter(params.get("convs", []))
    proj_iter = iter(params.get("projs", []))
    for k, step in enumerate(graph):
        if step in ("gn", "gn_silu"):
            h, fresh = gn_async(h, state["stats"][k], P, i, params["G"], params.get("eps", 1e-5),
                                gn_mode, params.get("gamma"), params.get("beta"),
                                "silu" if step == "gn_silu" else None)
            new_stats[k][i] = fresh
        elif step in ("attn_proj", "attn_proj_res"):
            tok = h.reshape(B, hb * W, C)
            ks_ = np.asarray(state["maps"][(k, "k")], dtype=F64).reshape(B, H * W, C)
            vs_ = np.asarray(state["maps"][(k, "v")], dtype=F64).reshape(B, H * W, C)
            out, kf, vf = attention_proj_splice(tok, next(proj_iter), ks_, vs_, H, W, P, i,
                                                params["heads"], params.get("scale"))
            new_maps[(k, "k")] = stale_update(new_maps[(k, "k")], kf.reshape(B, hb, W, C), P, i)
            new_maps[(k, "v")] = stale_update(new_maps[(k, "v")], vf.reshape(B, hb, W, C), P, i)
            h = out.reshape(B, hb, W, C)
            if step == "attn_proj_res":
                h = h + x_in
        elif step in ("conv", "conv_res"):
            w, bias = next(conv_iter)
            out = conv3x3_halo(h, state["maps"][k], w, bias, P, i)
            new_maps[k] = stale_update(new_maps[k], h, P, i)
            h = out + x_in if step == "conv_res" else out
        elif step == "attn":
            tok = h.reshape(B, hb * W, C)
            stale_tok = np.asarray(state["maps"][k], dtype=F64).reshape(B, H * W, C)
            out = attention_splice(tok, tok, tok, stale_tok, stale_tok, H, W, P, i,
                                   params["heads"], params.get("scale"))
            new_maps[k] = stale_update(new_maps[k], h, P, i)
            h = out.reshape(B, hb, W, C)
        else:
            raise ValueError(f"unknown step {step!r}")
        outputs.append(h)
    return outputs, {"stats": new_stats, "maps": new_maps}


def displaced_step_all(graph, params, x_full, state, P, gn_mode=GN_CORRECTED):
    """One denoising step of a layer with every patch displaced.

    study.space page, Method: each device computes only its own patch, using
    the previous step's activations as the context of the other patches;
    DistriFusion summary (atlas.scime.ai), Approach: the fresh activations are
    gathered to every device and become the next step's context.  So every
    patch i runs ``displaced_layer`` against the same previous-step ``state``,
    and the next state holds every patch's fresh band of each conv/attention
    input map and every patch's fresh GroupNorm moments (per GroupNorm step).

    Returns (outputs, next_state): outputs is every graph step's full-map
    output [B][H][W][C] (float64, patches side by side).
    """
    x = np.asarray(x_full, dtype=F64)
    B, H, W, C = x.shape
    h = H // P
    outputs = [np.empty((B, H, W, C), dtype=F64) for _ in graph]
    next_stats = {k: np.array(t, dtype=F64, copy=True) for k, t in state["stats"].items()}
    for i in range(P):
        outs, new_state = displaced_layer(graph, params, x[:, i * h:(i + 1) * h], state, P, i, gn_mode)
        for k, o in enumerate(outs):
            outputs[k][:, i * h:(i + 1) * h] = o
        for k in next_stats:
            next_stats[k][i] = new_state["stats"][k][i]
    inputs = [x] + outputs[:-1]
    next_maps = {}
    proj_iter = iter(params.get("projs", []))
    for k, step in enumerate(graph):
        if step in ("conv", "conv_res", "attn"):
            next_maps[k] = np.array(inputs[k], copy=True)
        elif step in ("attn_proj", "attn_proj_res"):
            wq, bq, wk, bk, wv, bv, wo, bo = next(proj_iter)
            next_maps[(k, "k")] = linear(inputs[k], wk, bk)
            next_maps[(k, "v")] = linear(inputs[k], wv, bv)
    return outputs, {"stats": next_stats, "maps": next_maps}
