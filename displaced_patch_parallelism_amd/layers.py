"""One layer's GPU state and its steps, composed from the four C-ABI calls.

A layer (``configs.LayerConfig``) owns, on the GPU:
  * for every GroupNorm step of its graph, that step's statistics table
    [P][B][G][2] of the previous step (each GroupNorm site normalises a
    different map, so each keeps its own table),
  * for every conv or attention step of its graph, the previous step's full
    input map [B][H][W][C] (the stale context; for attention it is the K/V
    map, since Q = K = V = the step's input), and
  * for every attention step with learned projections ("attn_proj",
    "attn_proj_res"), the previous step's projected K and V maps (the K/V
    cache).
The residual steps "conv_res" and "attn_proj_res" add the layer's own input
patch to their output (the skip connection of a ResNet or transformer block),
inside the conv's or the output projection's epilogue.

``warmup(x)`` runs a synchronous step on the full map, patch by patch, and
leaves the state equal to that step's statistics and maps (warm-up steps are
synchronous: DistriFusion summary on atlas.scime.ai, warm-up rows of
"Measured effects reported in the paper").  ``step(x_patch, i)`` runs patch
i's displaced step against the state and then splices the patch's fresh
statistics and bands into it (on one GPU this stands for the patch's part of
the AllGather that refreshes every device's context for the next step).
"""

from typing import Dict, List, Optional, Sequence, Tuple

import torch

from . import (Patch, _dtype_code, dp_attention_splice, dp_conv3x3_halo, dp_conv3x3_halo_packed,
               dp_conv3x3_halo_residual, dp_conv3x3_pack_weights, dp_groupnorm_async, dp_groupnorm_conv3x3_halo,
               dp_linear, dp_linear_qkv, dp_linear_residual, dp_stale_update, dp_stats_update, workspace_bytes)

GN_STEPS = ("gn", "gn_silu")
CONV_STEPS = ("conv", "conv_res")
PROJ_STEPS = ("attn_proj", "attn_proj_res")
MAP_STEPS = CONV_STEPS + ("attn",)     # steps whose stale context is their own input map


def torch_dtype(name):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def _mark(events, name):
    if events is None:
        return None
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    events.setdefault(name, []).append((start, end))
    return end


def _done(end):
    if end is not None:
        end.record()


class DisplacedLayer:
    def __init__(self, cfg, convs: Sequence[Tuple["np.ndarray", "np.ndarray"]], device="cuda",  # noqa: F821
                 projs=None, fuse=False):
        self.cfg = cfg
        # fuse: a GroupNorm step that feeds a conv runs as one dp_groupnorm_conv3x3_halo call when
        # the state is refreshed in place (else as its two calls)
        self.fuse = fuse
        self.device = torch.device(device)
        self.dt = torch_dtype(cfg.dtype)
        self.convs = [(torch.as_tensor(w).to(self.device, self.dt).contiguous(),
                       torch.as_tensor(b).to(self.device, torch.float32).contiguous()) for w, b in convs]
        # bf16 conv weights are packed once into the layout the kernels read as whole cache lines
        self.wpacked = [dp_conv3x3_pack_weights(w) if self.dt == torch.bfloat16 else None for w, _ in self.convs]
        # per attn_proj step: (wq, bq, wk, bk, wv, bv, wo, bo), weights in the storage type
        self.projs = [tuple(torch.as_tensor(a).to(self.device, self.dt if j % 2 == 0 else torch.float32).contiguous()
                            for j, a in enumerate(pr)) for pr in (projs or [])]
        # and W_q, W_k, W_v stacked [3C][C] with their biases [3C]: the three input projections
        # run as one dp_linear_qkv launch
        self.qkv = [(torch.cat([pr[0], pr[2], pr[4]]).contiguous(), torch.cat([pr[1], pr[3], pr[5]]).contiguous())
                    for pr in self.projs]
        c = cfg
        # one statistics table and one fresh-moments buffer per GroupNorm step
        self.tables: Dict = {k: torch.zeros((c.P, c.B, c.G, 2), dtype=torch.float32, device=self.device)
                             for k, s in enumerate(c.graph) if s in GN_STEPS}
        self.fresh = {k: torch.empty((c.B, c.G, 2), dtype=torch.float32, device=self.device)
                      for k in self.tables}
        full = (c.B, c.H, c.W, c.C)
        self.maps: Dict = {k: torch.zeros(full, dtype=self.dt, device=self.device)
                           for k, s in enumerate(c.graph) if s in MAP_STEPS}
        for k, s in enumerate(c.graph):
            if s in PROJ_STEPS:
                self.maps[(k, "k")] = torch.zeros(full, dtype=self.dt, device=self.device)
                self.maps[(k, "v")] = torch.zeros(full, dtype=self.dt, device=self.device)
        # patch-sized intermediates, reused by every step
        band = (c.B, c.h, c.W, c.C)
        self.bufs = [torch.empty(band, dtype=self.dt, device=self.device) for _ in c.graph]
        # attn_proj scratch bands: projected queries, attention output, fresh K and V (when
        # they are not written straight into the cache)
        self.pbufs = {k: {n: torch.empty(band, dtype=self.dt, device=self.device) for n in "qakv"}
                      for k, s in enumerate(c.graph) if s in PROJ_STEPS}
        # one workspace for every call of a step (calls are ordered on one stream); owned by the
        # layer so a captured graph keeps pointing at live memory
        code = _dtype_code(self.bufs[0])
        need = 0
        for w, _ in self.convs:
            need = max(need, workspace_bytes("conv", self.patch(0), code, int(w.shape[0])))
        conv_j = 0
        for k, s in enumerate(c.graph):
            if s in GN_STEPS:
                need = max(need, workspace_bytes("groupnorm", self.patch(0), code, c.G))
                if k + 1 < len(c.graph) and c.graph[k + 1] in CONV_STEPS:
                    need = max(need, workspace_bytes("groupnorm_conv", self.patch(0), code, c.G,
                                                     int(self.convs[conv_j][0].shape[0])))
            elif s in CONV_STEPS:
                conv_j += 1
            elif s == "attn" or s in PROJ_STEPS:
                need = max(need, workspace_bytes("attention", self.patch(0), code, c.heads, c.C // c.heads))
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)

    def patch(self, i) -> Patch:
        c = self.cfg
        return Patch(c.B, c.H, c.W, c.C, c.P, i)

    def band(self, full, j):
        h = self.cfg.h
        return full[:, j * h:(j + 1) * h].contiguous()

    def _tok(self, t):
        return t.reshape(t.shape[0], -1, t.shape[-1])

    @property
    def table(self):
        """The statistics table of the graph's first GroupNorm step."""
        return self.tables[min(self.tables)]

    def _conv(self, p, x_patch, stale, j, y_patch=None, ws=None, residual=None):
        """The layer's j-th conv (on its packed weights when they exist), plus a residual."""
        w, b = self.convs[j]
        if residual is not None:
            wp = self.wpacked[j]
            return dp_conv3x3_halo_residual(p, x_patch, stale, w if wp is None else wp, b, residual,
                                            y_patch=y_patch, packed=wp is not None, ws=ws)
        if self.wpacked[j] is not None:
            return dp_conv3x3_halo_packed(p, x_patch, stale, self.wpacked[j], b, y_patch=y_patch, ws=ws)
        return dp_conv3x3_halo(p, x_patch, stale, w, b, y_patch=y_patch, ws=ws)

    # ---- one patch, displaced ------------------------------------------------
    def calls(self, x_patch, i, gn_mode="corrected", update_state=True):
        """Patch i's displaced layer step as a list of (name, launch, outputs): each launch
        enqueues one C-ABI call on the current stream; ``outputs`` are the graph steps' patch
        outputs that call completes (none, one, or -- for a GroupNorm fused with its conv --
        two).  Running them in order is one step (without the splice of ``step`` when the
        state is not refreshed in place)."""
        c = self.cfg
        p = self.patch(i)
        in_place = update_state and c.B == 1 and gn_mode == "corrected"
        h = x_patch
        out_list = []
        conv_i = 0
        proj_i = 0
        fused_next = False
        for k, s in enumerate(c.graph):
            nxt = k + 1
            if in_place and nxt < len(c.graph) and nxt in self.maps:
                out = self.maps[nxt][:, i * c.h:(i + 1) * c.h]      # contiguous for B == 1
            else:
                out = self.bufs[k]
            if fused_next:           # this conv ran inside the GroupNorm call before it
                fused_next = False
                conv_i += 1
                h = out
                continue
            if (s in GN_STEPS and in_place and self.fuse and nxt < len(c.graph) and c.graph[nxt] in CONV_STEPS):
                # GroupNorm (+SiLU) and the conv it feeds in one call: the normalised band goes
                # straight into band i of the conv's stale map (``out``), the conv's output to
                # the conv step's own output
                table = self.tables[k]
                act = "silu" if s == "gn_silu" else None
                cout_k = nxt + 1
                y = self.maps[cout_k][:, i * c.h:(i + 1) * c.h] if cout_k < len(c.graph) and cout_k in self.maps \
                    else self.bufs[nxt]
                res = x_patch if c.graph[nxt] == "conv_res" else None
                w, b = self.convs[conv_i]
                wp = self.wpacked[conv_i]
                fn = (lambda h=h, y=y, table=table, act=act, res=res, w=w if wp is None else wp, b=b,
                      u=self.maps[nxt]: dp_groupnorm_conv3x3_halo(
                          p, h, c.G, u, w, b, stale_stats=table, eps=c.eps, mode=gn_mode, act=act,
                          fresh_stats_out=table[i], residual=res, y_patch=y, packed=wp is not None, ws=self.ws))
                out_list.append((f"{s}+{c.graph[nxt]}", fn, (out, y)))
                fused_next = True
                h = out
                continue
            if s in GN_STEPS:
                table = self.tables[k]
                stats = table[i] if in_place else self.fresh[k]
                act = "silu" if s == "gn_silu" else None
                fn = (lambda h=h, out=out, stats=stats, act=act, table=table: dp_groupnorm_async(
                    p, h, c.G, table, c.eps, gn_mode, act, fresh_stats_out=stats, y_patch=out, ws=self.ws))
            elif s in CONV_STEPS:
                res = x_patch if s == "conv_res" else None
                fn = (lambda h=h, out=out, k=k, j=conv_i, res=res: self._conv(p, h, self.maps[k], j, y_patch=out,
                                                                           ws=self.ws, residual=res))
                conv_i += 1
            elif s == "attn":
                tok, st, o = self._tok(h), self._tok(self.maps[k]), self._tok(out)
                fn = (lambda tok=tok, st=st, o=o: dp_attention_splice(
                    p, c.heads, tok, tok, tok, st, st, o_patch=o, ws=self.ws))
            else:   # attn_proj
                wo, bo = self.projs[proj_i][6:]
                proj_i += 1
                pb = self.pbufs[k]
                kcache, vcache = self.maps[(k, "k")], self.maps[(k, "v")]
                if in_place:       # fresh K and V straight into band i of the cache
                    kb = self._tok(kcache[:, i * c.h:(i + 1) * c.h])
                    vb = self._tok(vcache[:, i * c.h:(i + 1) * c.h])
                else:
                    kb, vb = self._tok(pb["k"]), self._tok(pb["v"])
                tok, q, a = self._tok(h), self._tok(pb["q"]), self._tok(pb["a"])
                w3, b3 = self.qkv[proj_i - 1]
                out_list.append(("proj_qkv", lambda tok=tok, q=q, kb=kb, vb=vb, w3=w3, b3=b3:
                                 dp_linear_qkv(tok, w3, b3, yq=q, yk=kb, yv=vb), ()))
                out_list.append(("attn", lambda q=q, kb=kb, vb=vb, a=a, ks=self._tok(kcache), vs=self._tok(vcache):
                                 dp_attention_splice(p, c.heads, q, kb, vb, ks, vs, o_patch=a, ws=self.ws), ()))
                if s == "attn_proj_res":
                    fn = (lambda a=a, o=self._tok(out), w=wo, b=bo, r=self._tok(x_patch):
                          dp_linear_residual(a, w, b, r, y=o))
                else:
                    fn = (lambda a=a, o=self._tok(out), w=wo, b=bo: dp_linear(a, w, b, y=o))
                s = "proj_o"
            out_list.append((s, fn, (out,)))
            h = out
        if in_place and 0 in self.maps:
            # a graph that starts with a conv or attention: its stale map's band i is the layer
            # input itself, which no earlier call wrote in place
            out_list.append(("stale_update", lambda: dp_stale_update(p, x_patch, self.maps[0]), ()))
        return out_list

    def step(self, x_patch, i, gn_mode="corrected", update_state=True, events=None) -> List[torch.Tensor]:
        """Patch i's displaced layer step; returns every graph step's patch output.

        With ``update_state`` (and B == 1, CORRECTED GroupNorm) each step that
        feeds a conv or attention writes its output straight into band i of that
        consumer's resident stale map, and the fresh moments go straight into
        slot i of the table: the state is refreshed with no separate splice.
        A patch never reads its own band of a stale map (the conv reads only the
        rows next to the band, the attention splices its fresh band in), so the
        in-place write is safe within the step.  Otherwise the outputs go to
        scratch buffers and, with ``update_state``, are spliced in afterwards.

        ``events``: optional dict; when given, each call is bracketed by a pair of
        torch.cuda.Event recorded on the current stream (the stream the library
        launches on), appended to events[name] as (start, end).
        """
        c = self.cfg
        in_place = update_state and c.B == 1 and gn_mode == "corrected"
        outs = []
        for s, fn, done in self.calls(x_patch, i, gn_mode, update_state):
            ev = _mark(events, s)
            fn()
            _done(ev)
            outs.extend(done)
        if update_state and not in_place:
            self.splice_state(i, x_patch, outs, events)
        return outs

    def capture(self, x_patch, i, gn_mode="corrected", update_state=True, steps=1):
        """``steps`` consecutive steps captured as one HIP graph (torch.cuda.CUDAGraph);
        replaying it repeats them on the same buffers with no host launch cost (a graph
        launch has a fixed cost of its own, which several steps per graph amortise)."""
        side = torch.cuda.Stream(self.device)
        side.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(side):
            for _ in range(2):
                self.step(x_patch, i, gn_mode, update_state)
        torch.cuda.current_stream(self.device).wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(steps):
                self.step(x_patch, i, gn_mode, update_state)
        return graph

    def step_all(self, x_full, gn_mode="corrected") -> List[torch.Tensor]:
        """Every patch's displaced step of one denoising step; returns each graph step's
        full-map output.

        Every patch reads the state the previous step left (the stale context is the
        previous step's for all patches alike); the fresh bands and moments are gathered
        into a second set of buffers and become the state only after the last patch --
        on one GPU this stands for the exchange that refreshes every device's context.
        ``gn_mode`` "corrected", "local" or "stale" selects the GroupNorm statistics.
        """
        c = self.cfg
        full = (c.B, c.H, c.W, c.C)
        outs_full = [torch.empty(full, dtype=self.dt, device=self.device) for _ in c.graph]
        next_tables = {k: torch.empty_like(t) for k, t in self.tables.items()}
        next_kv = {key: torch.empty(full, dtype=self.dt, device=self.device)
                   for key in self.maps if isinstance(key, tuple)}
        for i in range(c.P):
            p = self.patch(i)
            outs = self.step(self.band(x_full, i), i, gn_mode, update_state=False)
            for k, o in enumerate(outs):
                dp_stale_update(p, o, outs_full[k])
            for (k, kv), m in next_kv.items():
                dp_stale_update(p, self.pbufs[k][kv], m)
            for k, t in next_tables.items():
                dp_stats_update(c.P, i, self.fresh[k], t)
        for k, t in next_tables.items():
            self.tables[k].copy_(t)
        inputs = [x_full] + outs_full[:-1]
        for key, m in self.maps.items():
            m.copy_(next_kv[key] if isinstance(key, tuple) else inputs[key])
        return outs_full

    def splice_state(self, i, x_patch, outs, events=None):
        """Write patch i's fresh statistics and consumer-input bands into the state."""
        c = self.cfg
        p = self.patch(i)
        inputs = [x_patch] + outs[:-1]
        for k, s in enumerate(c.graph):
            if s in GN_STEPS:
                ev = _mark(events, "stats_update")
                dp_stats_update(c.P, i, self.fresh[k], self.tables[k])
            elif s in PROJ_STEPS:
                ev = _mark(events, "stale_update")
                dp_stale_update(p, self.pbufs[k]["k"], self.maps[(k, "k")])
                dp_stale_update(p, self.pbufs[k]["v"], self.maps[(k, "v")])
            elif k in self.maps:
                ev = _mark(events, "stale_update")
                dp_stale_update(p, inputs[k], self.maps[k])
            else:
                continue
            _done(ev)

    # ---- all patches, synchronous (warm-up) --------------------------------------
    def warmup(self, x_full) -> List[torch.Tensor]:
        """Synchronous full-map step; leaves the state of that step.  Returns full-map outputs."""
        c = self.cfg
        h_full = x_full
        outs = []
        conv_i = 0
        proj_i = 0
        for k, s in enumerate(c.graph):
            out_full = torch.empty((c.B, c.H, c.W, c.C), dtype=self.dt, device=self.device)
            if s in GN_STEPS:
                table, fresh = self.tables[k], self.fresh[k]
                for j in range(c.P):
                    dp_groupnorm_async(self.patch(j), self.band(h_full, j), c.G, None, c.eps, "local",
                                       fresh_stats_out=fresh, stats_only=True)
                    dp_stats_update(c.P, j, fresh, table)
                for j in range(c.P):
                    y, _ = dp_groupnorm_async(self.patch(j), self.band(h_full, j), c.G, table, c.eps,
                                              "corrected", "silu" if s == "gn_silu" else None,
                                              fresh_stats_out=fresh)
                    dp_stale_update(self.patch(j), y, out_full)
            elif s in PROJ_STEPS:
                wo, bo = self.projs[proj_i][6:]
                proj_i += 1
                tok = self._tok(h_full)
                kc, vc = self.maps[(k, "k")], self.maps[(k, "v")]
                w3, b3 = self.qkv[proj_i - 1]
                q_full = torch.empty_like(h_full)
                dp_linear_qkv(tok, w3, b3, yq=self._tok(q_full), yk=self._tok(kc), yv=self._tok(vc))
                a_full = torch.empty_like(h_full)
                for j in range(c.P):
                    pj = self.patch(j)
                    qj, kj, vj = (self._tok(self.band(m, j)) for m in (q_full, kc, vc))
                    a = dp_attention_splice(pj, c.heads, qj, kj, vj, self._tok(kc), self._tok(vc))
                    dp_stale_update(pj, a.reshape(qj.shape[0], c.h, c.W, c.C), a_full)
                if s == "attn_proj_res":
                    dp_linear_residual(self._tok(a_full), wo, bo, self._tok(x_full), y=self._tok(out_full))
                else:
                    dp_linear(self._tok(a_full), wo, bo, y=self._tok(out_full))
            else:
                for j in range(c.P):
                    dp_stale_update(self.patch(j), self.band(h_full, j), self.maps[k])
                for j in range(c.P):
                    pj = self.patch(j)
                    xb = self.band(h_full, j)
                    if s in CONV_STEPS:
                        res = self.band(x_full, j) if s == "conv_res" else None
                        o = self._conv(pj, xb, self.maps[k], conv_i, residual=res)
                    else:
                        tok = self._tok(xb)
                        st = self._tok(self.maps[k])
                        o = dp_attention_splice(pj, c.heads, tok, tok, tok, st, st).reshape(xb.shape)
                    dp_stale_update(pj, o, out_full)
                if s in CONV_STEPS:
                    conv_i += 1
            outs.append(out_full)
            h_full = out_full
        return outs
