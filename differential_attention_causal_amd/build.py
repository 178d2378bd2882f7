"""Builds libdiffattn.so in place: hipcc for gfx950, one object per source.

    python differential_attention_causal_amd/build.py

(run as a script: importing the package would load the library it builds).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libdiffattn.so")
OBJDIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "--offload-arch=gfx950",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    # packed fp32 VALU forms stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    # keep MFMA accumulators in VGPRs: the O rescale and the epilogue touch them
    # with VALU ops, and AGPR accumulators cost a copy each way per key tile
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]
SOURCES = ["prefill.hip", "window.hip", "decode.hip", "rope.hip", "vtiles.hip", "backward.hip", "grouped.hip",
           "gdecode.hip", "api.cpp"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, src + ".o")
    lang = [] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [HIPCC] + COMMON + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
