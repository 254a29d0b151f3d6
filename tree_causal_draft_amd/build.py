"""Builds libjt.so (HIP, gfx950) in-tree with hipcc.

    python -m tree_causal_draft_amd.build

Every HIP source is compiled with packed-FP32 code generation switched off
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass warns that
it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libjt.so")
SOURCES = ["mask.hip", "topw.hip", "verify.hip", "attn.hip", "api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libjt)")


FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(BUILD, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *FLAGS, *lang, "-c", path, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        noise = [ln for ln in (res.stderr or "").splitlines() if "packed-fp32-ops" not in ln]
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(noise))
        if verbose and noise:
            print("\n".join(noise), file=sys.stderr)
        objs.append(obj)
    tmp = LIB + ".tmp"
    res = subprocess.run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
