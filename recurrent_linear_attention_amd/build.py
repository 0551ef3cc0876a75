"""Build the KDA HIP library (libkda.so) in-tree for gfx950 with hipcc.

    python recurrent_linear_attention_amd/build.py

(Run as a script: importing it through the package would first load the library it builds.)
"""
from __future__ import annotations

import os
import shlex
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libkda.so")

SOURCES = ["kda_pool.cpp", "kda_plan.cpp", "kda_step.hip", "kda_prefill.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # explicit fmaf only: keeps decode, verify and commit bit-identical to each other
    "-ffp-contract=off",
    # no packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results in ordinary VGPRs: the state pass works on its accumulators with VALU
    # instructions (decay, conversions) every chunk, which AGPRs would turn into register moves
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    """Compile every source into ``lib/libkda.so``; returns its path. Raises on failure."""
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, f"-I{INCLUDE}", f"-I{CSRC}",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(shlex.quote(c) for c in cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    noise = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
