"""Builds libmoe_mx4.so (the C ABI + HIP kernels for gfx950) in-tree with hipcc.

    python -m mxfp4_mixture_experts_route_amd.build      # or build() from Python

Every call recompiles all sources (objects go to _build/, compiled in parallel).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libmoe_mx4.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["capi.hip", "pack.hip", "route.hip", "bucket.hip", "gemv.hip", "gemm.hip", "combine.hip",
           "decode.hip", "decode_layer.hip", "timing.hip", "quant.hip",
           "router.hip", "probe.hip"]

# -packed-fp32-ops: no packed fp32 VALU ops (v_pk_fma_f32 and friends) anywhere in device code.
CFLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src: str, extra: list[str], build_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + CFLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, extra: list[str] | None = None, out_path: str = LIB_PATH,
          build_dir: str = BUILD_DIR, link_extra: list[str] | None = None) -> str:
    """Compile every source with CFLAGS + extra into build_dir and link out_path (by default
    the in-tree library the package loads)."""
    extra = list(extra or [])
    os.makedirs(build_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, build_dir), SOURCES))
    tmp = out_path + ".tmp"
    cmd = ([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + list(link_extra or []) +
           ["-o", tmp] + objs)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out_path)
    if verbose:
        print(f"built {out_path}")
    return out_path


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
