"""Builds libdp.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m displaced_patch_parallelism_amd.build

Every call recompiles every translation unit (in parallel) and relinks.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdp.so")

ARCH = os.environ.get("DP_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 VALU ops (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{INCLUDE}", f"-I{CSRC}",
]

SOURCES = ["dp_api.cpp", "k_splice.hip", "k_groupnorm.hip", "k_conv.hip", "k_attention.hip", "k_linear.hip"]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + COMMON + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n" + "\n".join(msgs))
    return obj, "\n".join(msgs)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    for _, msg in results:
        if msg.strip() and verbose:
            print(msg)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
