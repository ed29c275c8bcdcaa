"""Build libatomattn.so (the HIP kernels + C ABI) for gfx950 with hipcc.

Usage: python -m windowed_atom_attention_amd.build
Each csrc/*.hip compiles to an object under _build/ (in parallel), then one
hipcc link produces windowed_atom_attention_amd/libatomattn.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libatomattn.so")
BUILD = os.path.join(ROOT, "_build")
ARCH = os.environ.get("WAA_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    # no fast-math and no denormal flushing: sigmoid/SiLU tails down to the
    # subnormal range must survive
    "-fno-gpu-flush-denormals-to-zero", "-fno-fast-math",
    # packed fp32 VALU ops stay off (plain fp32 instructions only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wall",
    "-Wno-unused-command-line-argument", "-Wno-pass-failed",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = ["hipcc", "-c", src, "-o", obj] + FLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s%s" % (src, r.stdout, r.stderr))
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if err:
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(SRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc link failed:\n%s%s" % (r.stdout, r.stderr))
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build()
