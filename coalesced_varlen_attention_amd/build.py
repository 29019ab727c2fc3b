"""Build libzl.so (HIP kernels for gfx950 + the C-ABI host runtime) in-tree with hipcc.

Usage:  python -m coalesced_varlen_attention_amd.build   (or call build())
The shared library lands next to this file; objects go to ``_build/``.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libzl.so")
ARCH = "gfx950"

# Packed fp32 VALU forms are disabled for all device code.
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
                "-packed-fp32-ops", "-Wno-unused-command-line-argument"]
HOST_FLAGS = ["-x", "c++", "-O2", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__"]
# Per-file device flags. The backward kernels keep MFMA results in arch VGPRs (the vector
# code reads every score and gradient element; the accumulator-register form costs one move
# per element).
EXTRA_DEVICE_FLAGS = {"zl_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    if os.path.exists(cand):
        return cand
    found = shutil.which("hipcc")
    if not found:
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libzl.so")
    return found


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    rocm_inc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")
    if src.endswith(".hip"):
        flags = DEVICE_FLAGS + EXTRA_DEVICE_FLAGS.get(os.path.basename(src), [])
    else:
        flags = HOST_FLAGS + ["-I", rocm_inc]
    cmd = [_hipcc(), *flags, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source under csrc/ and link libzl.so; returns the library path."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
