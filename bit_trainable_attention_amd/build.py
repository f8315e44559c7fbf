"""Build libsagebwd.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Run as `python -m bit_trainable_attention_amd.build`; the package loads the result from
its own directory.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsagebwd.so")

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I", INCLUDE, "-I", CSRC,
    # packed fp32 VALU ops stay off (only ordinary float code)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # correctly rounded float32 division and square root, IEEE denormals
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Wall", "-Wno-unused-result",
]
# per-file extras: the prologue is specified operation by operation (no FMA contraction); the
# attention kernels take maxima of finite values only, so max needs no NaN-quieting of its inputs;
# the backward's MFMAs write VGPRs (the dQ pass otherwise lands its products in AGPRs and reads
# each one back with v_accvgpr_read before converting it: a third VALU op per element)
EXTRA = {"prologue.hip": ["-ffp-contract=off"],
         "backward.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"]}
SOURCES = ["api.cpp", "prologue.hip", "forward.hip", "backward.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = ["hipcc", *lang, *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    # every symbol must resolve (a missing kernel stub would otherwise only show at load time)
    import ctypes
    ctypes.CDLL(tmp, mode=os.RTLD_NOW | os.RTLD_LOCAL)
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True).stdout
    bad = [ln for ln in nm.splitlines() if "sagebwd" in ln]
    if bad:
        raise RuntimeError("unresolved library symbols:\n" + "\n".join(bad))
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
