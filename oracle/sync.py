"""Synchronous (full-image) layer, in float64 -- the oracle's reference for warm-up steps.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Warm-up steps of DistriFusion run synchronously (DistriFusion summary on
atlas.scime.ai, table "Measured effects reported in the paper": the warm-up
ablation rows; "Limitations": warm-up steps are needed for few-step
samplers).  A synchronous step is the plain layer on the whole map: exact
GroupNorm statistics, a zero-padded conv over the full image, attention over
all tokens.  Its per-band GroupNorm moments and the inputs of its conv and
attention steps are what the next (displaced) step reads as stale context.

This code path is written independently of ``displaced.py``: it works on the
whole map and never splices.
"""

import numpy as np

F64 = np.float64


def group_norm(x, G, eps=1e-5, gamma=None, beta=None, act=None):
    """Exact GroupNorm over a full map [B][H][W][C] (population variance)."""
    x = np.asarray(x, dtype=F64)
    B, H, W, C = x.shape
    xg = x.reshape(B, H * W, G, C // G)
    mu = xg.mean(axis=(1, 3), keepdims=True)
    var = ((xg - mu) ** 2).mean(axis=(1, 3), keepdims=True)
    y = ((xg - mu) / np.sqrt(var + eps)).reshape(B, H, W, C)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=F64)
    if beta is not None:
        y = y + np.asarray(beta, dtype=F64)
    if act == "silu":
        y = y * (1.0 / (1.0 + np.exp(-y)))
    return y


def band_moments(x, G, P):
    """[P][B][G][2]: (E[x], E[x^2]) of each of the P row bands of a full map."""
    x = np.asarray(x, dtype=F64)
    B, H, W, C = x.shape
    h = H // P
    out = np.empty((P, B, G, 2), dtype=F64)
    for j in range(P):
        xg = x[:, j * h:(j + 1) * h].reshape(B, h * W, G, C // G)
        out[j, :, :, 0] = xg.mean(axis=(1, 3))
        out[j, :, :, 1] = (xg ** 2).mean(axis=(1, 3))
    return out


def conv3x3(x, w, bias):
    """Zero-padded 3x3 cross-correlation of a full map, stride 1."""
    x = np.asarray(x, dtype=F64)
    w = np.asarray(w, dtype=F64)
    B, H, W, C = x.shape
    padded = np.zeros((B, H + 2, W + 2, C), dtype=F64)
    padded[:, 1:-1, 1:-1] = x
    out = np.zeros((B, H, W, w.shape[0]), dtype=F64)
    for ky in range(3):
        for kx in range(3):
            out += padded[:, ky:ky + H, kx:kx + W, :] @ w[:, ky, kx, :].T
    if bias is not None:
        out += np.asarray(bias, dtype=F64)
    return out


def self_attention(x, heads, scale=None, chunk=512):
    """Full self-attention of a map with Q = K = V = x, heads split by channel."""
    x = np.asarray(x, dtype=F64)
    B, H, W, C = x.shape
    t = x.reshape(B, H * W, C)
    d = C // heads
    if scale is None or scale <= 0:
        scale = d ** -0.5
    out = np.empty_like(t)
    for b in range(B):
        for e in range(heads):
            sl = slice(e * d, (e + 1) * d)
            for s in range(0, H * W, chunk):
                S = scale * (t[b, s:s + chunk, sl] @ t[b, :, sl].T)
                S = S - S.max(axis=1, keepdims=True)
                E = np.exp(S)
                out[b, s:s + chunk, sl] = (E / E.sum(axis=1, keepdims=True)) @ t[b, :, sl]
    return out.reshape(B, H, W, C)


def attention(q, k, v, heads, scale=None, chunk=512):
    """softmax(scale * Q K^T) V per head over full maps [B][H][W][C] (no splice)."""
    q, k, v = (np.asarray(a, dtype=F64) for a in (q, k, v))
    B, H, W, C = q.shape
    tq, tk, tv = (a.reshape(B, H * W, C) for a in (q, k, v))
    d = C // heads
    if scale is None or scale <= 0:
        scale = d ** -0.5
    out = np.empty_like(tq)
    for b in range(B):
        for e in range(heads):
            sl = slice(e * d, (e + 1) * d)
            for s in range(0, H * W, chunk):
                S = scale * (tq[b, s:s + chunk, sl] @ tk[b, :, sl].T)
                S = S - S.max(axis=1, keepdims=True)
                E = np.exp(S)
                out[b, s:s + chunk, sl] = (E / E.sum(axis=1, keepdims=True)) @ tv[b, :, sl]
    return out.reshape(B, H, W, C)


def project(x, w, bias):
    """x W^T + bias over the channel axis of a map."""
    y = np.asarray(x, dtype=F64) @ np.asarray(w, dtype=F64).T
    return y + np.asarray(bias, dtype=F64) if bias is not None else y


def sync_layer(graph, params, x, P, state_only=False):
    """Run the layer on the full map; returns (outputs, state) for the next step.

    ``state_only``: stop once the last step's state entries are recorded, without computing
    its output (the state a displaced step reads never depends on the layer's final output);
    outputs then holds every step but the last.

    Graph steps: "gn", "gn_silu", "conv", "attn", "attn_proj", and the residual forms
    "conv_res" / "attn_proj_res" whose output adds the layer's own input x (the skip
    connection of a ResNet or transformer block).
    outputs: every step's full-map output.  state: "stats" = {step index: per-band moments
    [P][B][G][2] of that GroupNorm step's input} (every GroupNorm site keeps its own table),
    "maps" = {step index: full input map of that conv or attention step; (step index,
    "k"/"v"): the projected K / V maps of an attn_proj step}.
    """
    x = np.asarray(x, dtype=F64)
    h = x
    outputs = []
    state = {"stats": {}, "maps": {}}
    conv_iter = iter(params.get("convs", []))
    proj_iter = iter(params.get("projs", []))
    for k, step in enumerate(graph):
        last = k == len(graph) - 1
        if state_only and last:
            if step in ("gn", "gn_silu"):
                state["stats"][k] = band_moments(h, params["G"], P)
            elif step in ("attn_proj", "attn_proj_res"):
                wq, bq, wk, bk, wv, bv, wo, bo = next(proj_iter)
                state["maps"][(k, "k")] = project(h, wk, bk)
                state["maps"][(k, "v")] = project(h, wv, bv)
            elif step in ("conv", "conv_res", "attn"):
                state["maps"][k] = h
            else:
                raise ValueError(f"unknown step {step!r}")
            break
        if step in ("attn_proj", "attn_proj_res"):
            wq, bq, wk, bk, wv, bv, wo, bo = next(proj_iter)
            q, kk, vv = project(h, wq, bq), project(h, wk, bk), project(h, wv, bv)
            state["maps"][(k, "k")] = kk
            state["maps"][(k, "v")] = vv
            h = project(attention(q, kk, vv, params["heads"], params.get("scale")), wo, bo)
            if step == "attn_proj_res":
                h = h + x
            outputs.append(h)
            continue
        if step in ("gn", "gn_silu"):
            state["stats"][k] = band_moments(h, params["G"], P)
            h = group_norm(h, params["G"], params.get("eps", 1e-5), params.get("gamma"),
                           params.get("beta"), "silu" if step == "gn_silu" else None)
        elif step in ("conv", "conv_res"):
            w, bias = next(conv_iter)
            state["maps"][k] = h
            h = conv3x3(h, w, bias)
            if step == "conv_res":
                h = h + x
        elif step == "attn":
            state["maps"][k] = h
            h = self_attention(h, params["heads"], params.get("scale"))
        else:
            raise ValueError(f"unknown step {step!r}")
        outputs.append(h)
    return outputs, state
