"""displaced_patch_parallelism_amd -- the displaced-patch layer hot path on MI355X.

Thin ctypes binding of ``libdp.so`` (C ABI in ``include/dp.h``).  The
functions take torch tensors on a ROCm device, check device, dtype, shape and
contiguity, and pass raw pointers plus the current HIP stream to the library.
Every step of the computation runs in the library's HIP kernels; there is no
fallback: if the library is not built, or a tensor is not on a GPU, the call
raises.

Patch geometry: ``Patch(B, H, W, C, P, i)`` -- full NHWC map [B][H][W][C],
P equal row bands, this call computes band i (rows i*H/P .. (i+1)*H/P).
"""

import ctypes
import os
from typing import NamedTuple, Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdp.so")

DP_OK, DP_ERR_ARG, DP_ERR_UNSUPPORTED, DP_ERR_HIP = 0, 1, 2, 3
DP_F32, DP_BF16 = 0, 1
GN_MODES = {"corrected": 0, "local": 1, "stale": 2}
ACTS = {None: 0, "none": 0, "silu": 1}


class DpError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"dp status {status}: {msg}")
        self.status = status


class Patch(NamedTuple):
    B: int
    H: int
    W: int
    C: int
    P: int
    i: int

    @property
    def h(self):
        return self.H // self.P

    @property
    def r0(self):
        return self.i * (self.H // self.P)


class _CPatch(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "H", "W", "C", "P", "i")]


_lib = None


def lib():
    """The loaded libdp.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "or python -m displaced_patch_parallelism_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_float
        pp = ctypes.POINTER(_CPatch)
        psz = ctypes.POINTER(ctypes.c_size_t)
        sigs = {
            "dp_groupnorm_async_ws": [pp, i32, i32, psz],
            "dp_groupnorm_async": [pp, i32, i32, f32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "dp_groupnorm_async_noalloc": [pp, i32, i32, f32, i32, i32, vp, vp, vp, vp, vp, vp, vp],
            "dp_conv3x3_halo_ws": [pp, i32, i32, psz],
            "dp_conv3x3_halo": [pp, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp],
            "dp_conv3x3_pack_weights": [i32, i32, i32, vp, vp, vp],
            "dp_conv3x3_halo_packed": [pp, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp],
            "dp_attention_splice_ws": [pp, i32, i32, i32, psz],
            "dp_attention_splice": [pp, i32, i32, i32, f32, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "dp_stale_update": [pp, i32, vp, vp, vp],
            "dp_linear": [i32, i32, i32, i32, vp, ctypes.c_int64, vp, vp, vp, ctypes.c_int64, vp],
            "dp_conv3x3_halo_residual": [pp, i32, i32, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp],
            "dp_linear_residual": [i32, i32, i32, i32, vp, ctypes.c_int64, vp, vp, vp, ctypes.c_int64, vp,
                                   ctypes.c_int64, vp],
            "dp_linear_qkv": [i32, i32, i32, i32, vp, ctypes.c_int64, vp, vp, vp, ctypes.c_int64, vp,
                              ctypes.c_int64, vp, ctypes.c_int64, vp],
            "dp_groupnorm_conv3x3_halo_ws": [pp, i32, i32, i32, psz],
            "dp_groupnorm_conv3x3_halo": [pp, i32, i32, f32, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp, i32, vp,
                                          vp, vp, vp, sz, vp],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.dp_conv3x3_packed_weights_bytes.argtypes = [i32, i32]
        L.dp_conv3x3_packed_weights_bytes.restype = sz
        L.dp_last_error.restype = ctypes.c_char_p
        L.dp_last_error.argtypes = []
        L.dp_version.restype = ctypes.c_char_p
        L.dp_version.argtypes = []
        _lib = L
    return _lib


def _check(status):
    if status != DP_OK:
        raise DpError(status, lib().dp_last_error().decode())


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DP_BF16
    if t.dtype == torch.float32:
        return DP_F32
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t, name, shape=None, dtype=None, device=None):
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a ROCm GPU device (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream(device):
    return _torch().cuda.current_stream(device).cuda_stream


def _cpatch(p: Patch):
    return ctypes.byref(_CPatch(*[int(v) for v in p]))


_ws_cache = {}


def _workspace(nbytes, device, ws):
    """Caller workspace if given, else a buffer cached per (device, stream).

    Calls on one stream run in order, so they can share scratch; calls on two streams may
    run at once, so each stream gets its own.  The buffer is allocated on the stream that
    uses it: when a larger one replaces it, the caching allocator hands the old memory out
    again only after the work already queued on that stream.  Code captured into a HIP graph
    should pass `ws` explicitly, so that the graph keeps pointing at memory it owns."""
    torch = _torch()
    if nbytes == 0:
        return None, 0
    if ws is not None:
        return ws.data_ptr(), ws.numel() * ws.element_size()
    stream = torch.cuda.current_stream(device)
    key = (device.type, device.index, stream.cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        with torch.cuda.stream(stream):
            buf = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf.data_ptr(), buf.numel()


def workspace_bytes(kind, patch: Patch, dtype_code, *args):
    """Bytes of workspace an entry point needs ("groupnorm", "conv", "attention")."""
    out = ctypes.c_size_t(0)
    fn = {"groupnorm": lib().dp_groupnorm_async_ws, "conv": lib().dp_conv3x3_halo_ws,
          "attention": lib().dp_attention_splice_ws, "groupnorm_conv": lib().dp_groupnorm_conv3x3_halo_ws}[kind]
    _check(fn(_cpatch(patch), dtype_code, *args, ctypes.byref(out)))
    return out.value


def dp_stale_update(patch: Patch, x_patch, stale):
    """stale[:, r0:r0+h] = x_patch, bit for bit (in place)."""
    p = Patch(*patch)
    dt = _dtype_code(stale)
    _ptr(stale, "stale", (p.B, p.H, p.W, p.C))
    _ptr(x_patch, "x_patch", (p.B, p.h, p.W, p.C), stale.dtype, stale.device)
    _check(lib().dp_stale_update(_cpatch(p), dt, x_patch.data_ptr(), stale.data_ptr(), _stream(stale.device)))
    return stale


def dp_stats_update(P, i, fresh_stats, table):
    """Copy one patch's GroupNorm moments [B][G][2] into slot i of the [P][B][G][2] table."""
    torch = _torch()
    if table.dtype != torch.float32 or fresh_stats.dtype != torch.float32:
        raise TypeError("statistics are float32")
    n = fresh_stats.numel()
    if table.numel() != P * n:
        raise ValueError("table must hold P slots of the statistics shape")
    p = Patch(1, P, 1, n, P, i)
    return dp_stale_update(p, fresh_stats.reshape(1, 1, 1, n), table.view(1, P, 1, n))


def dp_groupnorm_async(patch: Patch, x_patch, G, stale_stats=None, eps=1e-5, mode="corrected",
                       act=None, gamma=None, beta=None, fresh_stats_out=None, y_patch=None,
                       stats_only=False, ws=None):
    """Corrected asynchronous GroupNorm of patch i; returns (y_patch, fresh_stats_out)."""
    torch = _torch()
    p = Patch(*patch)
    dt = _dtype_code(x_patch)
    dev = x_patch.device
    _ptr(x_patch, "x_patch", (p.B, p.h, p.W, p.C))
    if fresh_stats_out is None:
        fresh_stats_out = torch.empty((p.B, G, 2), dtype=torch.float32, device=dev)
    if y_patch is None and not stats_only:
        y_patch = torch.empty_like(x_patch)
    _ptr(fresh_stats_out, "fresh_stats_out", (p.B, G, 2), torch.float32, dev)
    _ptr(y_patch, "y_patch", (p.B, p.h, p.W, p.C), x_patch.dtype, dev)
    _ptr(stale_stats, "stale_stats", (p.P, p.B, G, 2), torch.float32, dev)
    _ptr(gamma, "gamma", (p.C,), torch.float32, dev)
    _ptr(beta, "beta", (p.C,), torch.float32, dev)
    need = workspace_bytes("groupnorm", p, dt, G)
    wptr, wbytes = _workspace(need, dev, ws)
    gp = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    _check(lib().dp_groupnorm_async(
        _cpatch(p), dt, G, float(eps), GN_MODES[mode], ACTS[act], x_patch.data_ptr(), gp(stale_stats),
        gp(gamma), gp(beta), fresh_stats_out.data_ptr(), gp(y_patch), wptr, wbytes, _stream(dev)))
    return y_patch, fresh_stats_out


def dp_groupnorm_async_noalloc(patch: Patch, x_patch, G, stale_stats=None, eps=1e-5, mode="corrected",
                               act=None, gamma=None, beta=None, fresh_stats_out=None, y_patch=None,
                               stats_only=False):
    """dp_groupnorm_async without a workspace: the library's static scratch holds the partials (one
    array per GPU, shared by every call on it; calls that overlap on one GPU race).  The outputs
    must already exist when this is called from code that cannot allocate."""
    torch = _torch()
    p = Patch(*patch)
    dt = _dtype_code(x_patch)
    dev = x_patch.device
    _ptr(x_patch, "x_patch", (p.B, p.h, p.W, p.C))
    if fresh_stats_out is None:
        fresh_stats_out = torch.empty((p.B, G, 2), dtype=torch.float32, device=dev)
    if y_patch is None and not stats_only:
        y_patch = torch.empty_like(x_patch)
    _ptr(fresh_stats_out, "fresh_stats_out", (p.B, G, 2), torch.float32, dev)
    _ptr(y_patch, "y_patch", (p.B, p.h, p.W, p.C), x_patch.dtype, dev)
    _ptr(stale_stats, "stale_stats", (p.P, p.B, G, 2), torch.float32, dev)
    _ptr(gamma, "gamma", (p.C,), torch.float32, dev)
    _ptr(beta, "beta", (p.C,), torch.float32, dev)
    gp = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    _check(lib().dp_groupnorm_async_noalloc(
        _cpatch(p), dt, G, float(eps), GN_MODES[mode], ACTS[act], x_patch.data_ptr(), gp(stale_stats),
        gp(gamma), gp(beta), fresh_stats_out.data_ptr(), gp(y_patch), _stream(dev)))
    return y_patch, fresh_stats_out


def dp_conv3x3_halo(patch: Patch, x_patch, x_stale, w, bias=None, y_patch=None, ws=None):
    """3x3 conv of patch i with stale halo rows; returns y_patch [B][h][W][Cout]."""
    torch = _torch()
    p = Patch(*patch)
    dt = _dtype_code(x_patch)
    dev = x_patch.device
    cout = int(w.shape[0])
    _ptr(x_patch, "x_patch", (p.B, p.h, p.W, p.C))
    _ptr(x_stale, "x_stale", (p.B, p.H, p.W, p.C), x_patch.dtype, dev)
    _ptr(w, "w", (cout, 3, 3, p.C), x_patch.dtype, dev)
    _ptr(bias, "bias", (cout,), torch.float32, dev)
    if y_patch is None:
        y_patch = torch.empty((p.B, p.h, p.W, cout), dtype=x_patch.dtype, device=dev)
    _ptr(y_patch, "y_patch", (p.B, p.h, p.W, cout), x_patch.dtype, dev)
    need = workspace_bytes("conv", p, dt, cout)
    wptr, wbytes = _workspace(need, dev, ws)
    _check(lib().dp_conv3x3_halo(_cpatch(p), dt, cout, x_patch.data_ptr(), x_stale.data_ptr(), w.data_ptr(),
                                 None if bias is None else bias.data_ptr(), y_patch.data_ptr(), wptr, wbytes,
                                 _stream(dev)))
    return y_patch


def dp_conv3x3_pack_weights(w, w_packed=None):
    """bf16 conv weights [Cout][3][3][Cin] -> the packed layout [3][Cin/32][3][Cout][32] that
    dp_conv3x3_halo_packed reads as whole cache lines (pack once; weights are constant)."""
    torch = _torch()
    cout, cin = int(w.shape[0]), int(w.shape[3])
    _ptr(w, "w", (cout, 3, 3, cin))
    if cin % 64 or cout % 32:
        raise DpError(DP_ERR_UNSUPPORTED, f"packed weights need Cin % 64 == 0 and Cout % 32 == 0 "
                                          f"(Cin={cin}, Cout={cout})")
    shape = (3, cin // 32, 3, cout, 32)
    if w_packed is None:
        w_packed = torch.empty(shape, dtype=w.dtype, device=w.device)
    _ptr(w_packed, "w_packed", shape, w.dtype, w.device)
    _check(lib().dp_conv3x3_pack_weights(_dtype_code(w), cin, cout, w.data_ptr(), w_packed.data_ptr(),
                                         _stream(w.device)))
    return w_packed


def dp_conv3x3_halo_packed(patch: Patch, x_patch, x_stale, w_packed, bias=None, y_patch=None, ws=None):
    """dp_conv3x3_halo on packed weights (from dp_conv3x3_pack_weights); bitwise the same result."""
    torch = _torch()
    p = Patch(*patch)
    dt = _dtype_code(x_patch)
    dev = x_patch.device
    cout = int(w_packed.shape[3])
    _ptr(x_patch, "x_patch", (p.B, p.h, p.W, p.C))
    _ptr(x_stale, "x_stale", (p.B, p.H, p.W, p.C), x_patch.dtype, dev)
    _ptr(w_packed, "w_packed", (3, p.C // 32, 3, cout, 32), x_patch.dtype, dev)
    _ptr(bias, "bias", (cout,), torch.float32, dev)
    if y_patch is None:
        y_patch = torch.empty((p.B, p.h, p.W, cout), dtype=x_patch.dtype, device=dev)
    _ptr(y_patch, "y_patch", (p.B, p.h, p.W, cout), x_patch.dtype, dev)
    need = workspace_bytes("conv", p, dt, cout)
    wptr, wbytes = _workspace(need, dev, ws)
    _check(lib().dp_conv3x3_halo_packed(_cpatch(p), dt, cout, x_patch.data_ptr(), x_stale.data_ptr(),
                                        w_packed.data_ptr(), None if bias is None else bias.data_ptr(),
                                        y_patch.data_ptr(), wptr, wbytes, _stream(dev)))
    return y_patch


def dp_conv3x3_halo_residual(patch: Patch, x_patch, x_stale, w, bias=None, residual=None, y_patch=None,
                             packed=None, ws=None):
    """3x3 conv of patch i with stale halo rows plus a residual [B][h][W][Cout] added before
    rounding.  ``w`` is [Cout][3][3][Cin], or the packed layout of dp_conv3x3_pack_weights
    (detected from its 5-d shape unless ``packed`` says)."""
    torch = _torch()
    p = Patch(*patch)
    dt = _dtype_code(x_patch)
    dev = x_patch.device
    if packed is None:
        packed = w.dim() == 5
    cout = int(w.shape[3]) if packed else int(w.shape[0])
    wshape = (3, p.C // 32, 3, cout, 32) if packed else (cout, 3, 3, p.C)
    _ptr(x_patch, "x_patch", (p.B, p.h, p.W, p.C))
    _ptr(x_stale, "x_stale", (p.B, p.H, p.W, p.C), x_patch.dtype, dev)
    _ptr(w, "w", wshape, x_patch.dtype, dev)
    _ptr(bias, "bias", (cout,), torch.float32, dev)
    _ptr(residual, "residual", (p.B, p.h, p.W, cout), x_patch.dtype, dev)
    if y_patch is None:
        y_patch = torch.empty((p.B, p.h, p.W, cout), dtype=x_patch.dtype, device=dev)
    _ptr(y_patch, "y_patch", (p.B, p.h, p.W, cout), x_patch.dtype, dev)
    need = workspace_bytes("conv", p, dt, cout)
    wptr, wbytes = _workspace(need, dev, ws)
    gp = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    _check(lib().dp_conv3x3_halo_residual(_cpatch(p), dt, cout, x_patch.data_ptr(), x_stale.data_ptr(),
                                          w.data_ptr(), 1 if packed else 0, gp(bias), gp(residual),
                                          y_patch.data_ptr(), wptr, wbytes, _stream(dev)))
    return y_patch


def dp_groupnorm_conv3x3_halo(patch: Patch, x_patch, G, u_stale, w, bias=None, stale_stats=None, eps=1e-5,
                              mode="corrected", act=None, gamma=None, beta=None, fresh_stats_out=None,
                              residual=None, y_patch=None, packed=None, ws=None):
    """GroupNorm (+SiLU) of patch i, then the 3x3 conv with stale halo on the normalised band; band i
    of ``u_stale`` (the conv input's stale map) receives the normalised band.  ``w`` as in
    dp_conv3x3_halo_residual.  Returns (y_patch, fresh_stats_out)."""
    torch = _torch()
    p = Patch(*patch)
    dt = _dtype_code(x_patch)
    dev = x_patch.device
    if packed is None:
        packed = w.dim() == 5
    cout = int(w.shape[3]) if packed else int(w.shape[0])
    wshape = (3, p.C // 32, 3, cout, 32) if packed else (cout, 3, 3, p.C)
    _ptr(x_patch, "x_patch", (p.B, p.h, p.W, p.C))
    _ptr(u_stale, "u_stale", (p.B, p.H, p.W, p.C), x_patch.dtype, dev)
    _ptr(w, "w", wshape, x_patch.dtype, dev)
    _ptr(bias, "bias", (cout,), torch.float32, dev)
    _ptr(residual, "residual", (p.B, p.h, p.W, cout), x_patch.dtype, dev)
    if fresh_stats_out is None:
        fresh_stats_out = torch.empty((p.B, G, 2), dtype=torch.float32, device=dev)
    if y_patch is None:
        y_patch = torch.empty((p.B, p.h, p.W, cout), dtype=x_patch.dtype, device=dev)
    _ptr(fresh_stats_out, "fresh_stats_out", (p.B, G, 2), torch.float32, dev)
    _ptr(y_patch, "y_patch", (p.B, p.h, p.W, cout), x_patch.dtype, dev)
    _ptr(stale_stats, "stale_stats", (p.P, p.B, G, 2), torch.float32, dev)
    _ptr(gamma, "gamma", (p.C,), torch.float32, dev)
    _ptr(beta, "beta", (p.C,), torch.float32, dev)
    need = workspace_bytes("groupnorm_conv", p, dt, G, cout)
    wptr, wbytes = _workspace(need, dev, ws)
    gp = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    _check(lib().dp_groupnorm_conv3x3_halo(
        _cpatch(p), dt, G, float(eps), GN_MODES[mode], ACTS[act], x_patch.data_ptr(), gp(stale_stats), gp(gamma),
        gp(beta), fresh_stats_out.data_ptr(), u_stale.data_ptr(), cout, w.data_ptr(), 1 if packed else 0, gp(bias),
        gp(residual), y_patch.data_ptr(), wptr, wbytes, _stream(dev)))
    return y_patch, fresh_stats_out


def dp_attention_splice(patch: Patch, heads, q_patch, k_patch, v_patch, k_stale, v_stale, o_patch=None,
                        scale=0.0, ws=None):
    """Attention of patch i's queries over spliced K/V; tensors are token-major [B][tokens][C]."""
    torch = _torch()
    p = Patch(*patch)
    dt = _dtype_code(q_patch)
    dev = q_patch.device
    d = p.C // heads
    band = (p.B, p.h * p.W, p.C)
    full = (p.B, p.H * p.W, p.C)
    for t, n, s in ((q_patch, "q_patch", band), (k_patch, "k_patch", band), (v_patch, "v_patch", band),
                    (k_stale, "k_stale", full), (v_stale, "v_stale", full)):
        _ptr(t, n, s, q_patch.dtype, dev)
    if o_patch is None:
        o_patch = torch.empty(band, dtype=q_patch.dtype, device=dev)
    _ptr(o_patch, "o_patch", band, q_patch.dtype, dev)
    need = workspace_bytes("attention", p, dt, heads, d)
    wptr, wbytes = _workspace(need, dev, ws)
    _check(lib().dp_attention_splice(_cpatch(p), dt, heads, d, float(scale), q_patch.data_ptr(),
                                     k_patch.data_ptr(), v_patch.data_ptr(), k_stale.data_ptr(),
                                     v_stale.data_ptr(), o_patch.data_ptr(), wptr, wbytes, _stream(dev)))
    return o_patch


def dp_linear(x, w, bias=None, y=None):
    """y = x W^T + bias over the last axis.  x: [..., K] whose rows may be strided (the last axis
    contiguous, the leading axes collapsible to one row stride), w: [N][K] contiguous, bias: [N]
    float32 or None; y: [..., N] with the same row structure, allocated if None."""
    return _linear(x, w, bias, None, y)


def dp_linear_residual(x, w, bias=None, r=None, y=None):
    """y = x W^T + bias + r, the residual r [..., N] (rows as y) added before rounding."""
    return _linear(x, w, bias, r, y)


def _rows(t, name, width):
    """(rows, row stride) of a tensor read as rows of `width` contiguous elements: any leading
    shape whose rows form one strided sequence (a token-major map [B][tokens][C] included)."""
    if t.dim() < 1 or t.shape[-1] != width or (t.numel() and t.stride(-1) != 1):
        raise ValueError(f"{name} must end in a contiguous axis of {width}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    m = 1
    for d in t.shape[:-1]:
        m *= int(d)
    flat = t.reshape(m, width) if m else t
    if m and flat.data_ptr() != t.data_ptr():
        raise ValueError(f"{name} rows are not one strided sequence")
    ld = flat.stride(0) if m > 1 else width
    return m, ld


def dp_linear_qkv(x, w3, bias3=None, yq=None, yk=None, yv=None):
    """(x W_q^T + b_q, x W_k^T + b_k, x W_v^T + b_v) in one launch: w3 = [W_q; W_k; W_v] [3N][K],
    bias3 [3N] float32.  x and the outputs are read as rows like dp_linear's (e.g. token-major
    maps); missing outputs are allocated with x's leading shape."""
    torch = _torch()
    dt = _dtype_code(x)
    dev = x.device
    if w3.dim() != 2 or w3.shape[0] % 3:
        raise ValueError("w3 must be [3N][K]")
    N, K = int(w3.shape[0]) // 3, int(w3.shape[1])
    if x.shape[-1] != K:
        raise ValueError(f"x has {x.shape[-1]} columns, w3 expects {K}")
    _ptr(w3, "w3", (3 * N, K), x.dtype, dev)
    _ptr(bias3, "bias3", (3 * N,), torch.float32, dev)
    M, ldx = _rows(x, "x", K)
    outs, lds = [], []
    for name, y in (("yq", yq), ("yk", yk), ("yv", yv)):
        if y is None:
            y = torch.empty(tuple(x.shape[:-1]) + (N,), dtype=x.dtype, device=dev)
        if y.dtype != x.dtype or y.device != dev:
            raise TypeError(f"{name} must have x's dtype and device")
        My, ld = _rows(y, name, N)
        if My != M:
            raise ValueError(f"{name} has {My} rows, x has {M}")
        outs.append(y)
        lds.append(ld)
    bp = None if bias3 is None else bias3.data_ptr()
    _check(lib().dp_linear_qkv(dt, M, N, K, x.data_ptr(), ldx, w3.data_ptr(), bp, outs[0].data_ptr(), lds[0],
                               outs[1].data_ptr(), lds[1], outs[2].data_ptr(), lds[2], _stream(dev)))
    return tuple(outs)


def _linear(x, w, bias, r, y):
    torch = _torch()
    dt = _dtype_code(x)
    dev = x.device
    N, K = int(w.shape[0]), int(w.shape[1])
    if x.shape[-1] != K:
        raise ValueError(f"x has {x.shape[-1]} columns, w expects {K}")
    _ptr(w, "w", (N, K), x.dtype, dev)
    _ptr(bias, "bias", (N,), torch.float32, dev)
    if y is None:
        y = torch.empty(tuple(x.shape[:-1]) + (N,), dtype=x.dtype, device=dev)

    M, ldx = _rows(x, "x", K)
    My, ldy = _rows(y, "y", N)
    if My != M:
        raise ValueError(f"y has {My} rows, x has {M}")
    bp = None if bias is None else bias.data_ptr()
    if r is None:
        _check(lib().dp_linear(dt, M, N, K, x.data_ptr(), ldx, w.data_ptr(), bp, y.data_ptr(), ldy, _stream(dev)))
        return y
    if r.dtype != x.dtype or r.device != dev:
        raise TypeError("r must have x's dtype and device")
    Mr, ldr = _rows(r, "r", N)
    if Mr != M:
        raise ValueError(f"r has {Mr} rows, x has {M}")
    _check(lib().dp_linear_residual(dt, M, N, K, x.data_ptr(), ldx, w.data_ptr(), bp, r.data_ptr(), ldr,
                                    y.data_ptr(), ldy, _stream(dev)))
    return y


def version():
    return lib().dp_version().decode()
