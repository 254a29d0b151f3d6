"""Builds libjt.so (HIP, gfx950) in-tree with hipcc.

    python -m tree_causal_draft_amd.build

Every HIP source is compiled with packed-FP32 code generation switched off
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass warns that
it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libjt.so")
SOURCES = ["libjt.hip", "api.cpp"]  # libjt.hip includes every .hip file
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libjt)")


FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


# Kernels whose software pipeline counts outstanding loads exactly (s_waitcnt vmcnt(N)):
# a register spill would add scratch loads to that count, so the build refuses one.  The
# logit scans are held to the same rule: a spill there would sit in the streaming loop,
# beside the next piece's loads.
NO_SCRATCH = {"libjt.hip": ("attn_bf16_kernel", "step_phase1", "step_scan_kernel",
                            "topw_partial_kernel", "argmax_partial_kernel",
                            "sample_partial_kernel")}


def _scratch_violations(stderr: str, kernels):
    bad, fn = [], None
    for ln in stderr.splitlines():
        if "Function Name:" in ln:
            fn = ln.split("Function Name:")[1].split()[0]
        elif "ScratchSize [bytes/lane]:" in ln and fn and any(k in fn for k in kernels):
            if int(ln.split("ScratchSize [bytes/lane]:")[1].split()[0]) != 0:
                bad.append(fn)
    return bad


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(BUILD, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        extra = ["-Rpass-analysis=kernel-resource-usage"] if src in NO_SCRATCH else []
        cmd = [cc, *FLAGS, *extra, *lang, "-c", path, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        noise = [ln for ln in (res.stderr or "").splitlines()
                 if "packed-fp32-ops" not in ln and "remark:" not in ln
                 and not re.match(r"^\s*(\d+\s*)?\|", ln)]
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(noise))
        if src in NO_SCRATCH:
            bad = _scratch_violations(res.stderr or "", NO_SCRATCH[src])
            if bad:
                raise RuntimeError(f"{src}: kernels spill to scratch: {bad}")
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
