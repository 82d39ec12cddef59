"""Builds the gfx950 HIP library ``libmoe_mi355x.so`` in-tree with hipcc.

Every source is compiled for gfx950 only, with packed-fp32 instruction
selection turned off (-packed-fp32-ops), then linked into one shared library
that exports the C ABI of ``include/moe_mi355x.h``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
SOURCES = ["api.hip", "route_topk.hip", "permute.hip", "grouped_gemm.hip", "grouped_gemm_small.hip",
           "combine.hip", "quantize.hip", "backward.hip", "wgrad.hip", "router.hip", "probes.hip", "debug.hip", "fused_layer.hip",
           "tiled.hip"]
LIB_NAME = "libmoe_mi355x.so"
DEBUG_LIB_NAME = "libmoe_mi355x_debug.so"
ARCH = "gfx950"


def library_path(debug: bool = False) -> str:
    return os.path.join(PKG, DEBUG_LIB_NAME if debug else LIB_NAME)


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the MoE library needs ROCm's hipcc to build")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Wno-unused-command-line-argument",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include")]


def build(verbose: bool = False, resource_usage: bool = False, debug: bool = False) -> str:
    """Compiles every source and links the library. debug=True builds the debug
    library instead (MOE_DEBUG: device-side precondition checks; relocatable
    device code, so every kernel sees the one status word debug.hip defines)."""
    bdir = BUILD + ("_debug" if debug else "")
    os.makedirs(bdir, exist_ok=True)
    cc = hipcc()
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    if debug:
        extra += ["-DMOE_DEBUG", "-fgpu-rdc"]

    def compile_one(src):
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        cmd = [cc, *common_flags(), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        # hipcc's host pass does not know the gfx feature flag; that warning is harmless
        noise = "is not a recognized feature for this target"
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
        if msg.strip() and (verbose or resource_usage):
            print(msg, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    out = library_path(debug)
    tmp = out + f".tmp{os.getpid()}"
    link = ["-fgpu-rdc", "--hip-link"] if debug else []
    cmd = [cc, f"--offload-arch={ARCH}", *link, "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, resource_usage="--resource-usage" in sys.argv,
                debug="--debug" in sys.argv))
