"""Vendor-library references on the layer's contraction shapes (measurement only).

The conv is an implicit GEMM (M = B*h*W pixels, N = Cout, K = 9*Cin); the attention is
softmax(Q K^T) V per head over the whole map.  This times what the vendor libraries reach on
those shapes -- a plain bf16 GEMM through torch.matmul (hipBLASLt), and torch's fused
attention restricted to its flash / memory-efficient backends -- so that the library's kernels
can be compared with a known practical rate.  Nothing in the library calls these.

    python -m displaced_patch_parallelism_amd.diag.vendor_ref

prints one JSON line per shape.  Times are HIP-graph replays of back-to-back calls (an eager
loop where a library call cannot be captured; the line says which).
"""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)


def _time_us(fn, reps, replays=2):
    """GPU time per call: a HIP-graph replay of `reps` calls, or (when the library call cannot
    be captured) an eager loop of them; returns (us, how)."""
    import torch
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * replays), "graph"
    except RuntimeError:
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps * replays):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * replays), "eager"


def gemm_rows():
    import torch
    from displaced_patch_parallelism_amd.configs import CONFIGS
    shapes = [(n, c.B * c.Nq, c.C, 9 * c.C) for n, c in CONFIGS.items() if c.has_conv and c.dtype == "bf16"
              and n in ("c1", "c2", "c3", "c4a")]
    shapes.append(("square 8192", 8192, 8192, 8192))
    for name, M, N, K in shapes:
        a = torch.randn(M, K, device="cuda").to(torch.bfloat16)
        w = torch.randn(N, K, device="cuda").to(torch.bfloat16)     # weights [N][K], as the conv's
        wt = w.t()                                                   # a column-major K x N operand
        us, how = _time_us(lambda: a @ wt, reps=20)
        yield {"ref": "torch.matmul bf16", "shape": name, "M": M, "N": N, "K": K, "us": round(us, 2),
               "tflops": round(2.0 * M * N * K / us / 1e6, 1), "timing": how}


def attention_rows():
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    from displaced_patch_parallelism_amd.configs import CONFIGS
    for name in ("c2", "c3", "c4b"):
        c = CONFIGS[name]
        d = c.C // c.heads
        q = torch.randn(c.B, c.heads, c.Nq, d, device="cuda").to(torch.bfloat16)
        k = torch.randn(c.B, c.heads, c.N, d, device="cuda").to(torch.bfloat16)
        v = torch.randn(c.B, c.heads, c.N, d, device="cuda").to(torch.bfloat16)
        for label, backend in (("flash", SDPBackend.FLASH_ATTENTION), ("efficient", SDPBackend.EFFICIENT_ATTENTION)):
            row = {"ref": f"torch sdpa ({label})", "shape": name, "queries": c.Nq, "keys": c.N, "heads": c.heads}
            try:
                with sdpa_kernel([backend]):     # this backend only: no fallback to the math path
                    us, how = _time_us(lambda: F.scaled_dot_product_attention(q, k, v),
                                       reps=2 if name == "c4b" else 20)
                row.update(us=round(us, 2), tflops=round(c.attn_flops() / us / 1e6, 1), timing=how)
            except RuntimeError as e:            # backend not built for this device or shape
                row.update(error=str(e).splitlines()[0][:160])
            yield row


def main():
    import torch
    if not torch.cuda.is_available():
        print("needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    for row in gemm_rows():
        print(json.dumps(row), flush=True)
    for row in attention_rows():
        print(json.dumps(row), flush=True)


if __name__ == "__main__":
    main()
