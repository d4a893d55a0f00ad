"""Build libattn.so (gfx950) in-tree with hipcc.

    python -m exact_tiled_attention_attn_amd.build

Compiles the HIP kernels and the C ABI host code and links them into
``exact_tiled_attention_attn_amd/libattn.so`` next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libattn.so")

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall"]
# Packed fp32 VALU forms are kept out of the device code.  -fno-honor-nans:
# no value in the kernels is NaN unless an input is, and without it every
# fmax of an MFMA result first quiets a possible signaling NaN (one extra
# instruction per score).  Infinities (the -inf of masked scores) are kept.
DEVICE_ONLY = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "-fno-honor-nans"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libattn.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "not a recognized feature" not in line
                    and "argument unused during compilation" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}):\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = True) -> str:
    """Compile every source and link libattn.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for name in sorted(os.listdir(CSRC)):
        src = os.path.join(CSRC, name)
        if name.endswith(".hip"):
            flags = COMMON + DEVICE_ONLY + ["-x", "hip"]
        elif name.endswith(".cpp"):
            flags = COMMON
        else:
            continue
        obj = os.path.join(BUILD_DIR, name + ".o")
        _run([hipcc, *flags, "-c", src, "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-q" not in sys.argv)
    print(path)
