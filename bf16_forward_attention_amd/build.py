"""Ahead-of-time build of the HIP library for gfx950.

``python -m bf16_forward_attention_amd.build`` compiles
``csrc/attn_fwd.hip`` into ``libattn_fwd.so`` next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "attn_fwd.hip")
LIB = os.path.join(HERE, "libattn_fwd.so")
INCLUDE = os.path.join(ROOT, "include")

# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32.
# No fast-math: NaN/Inf propagation is part of the contract.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def build(verbose: bool = False) -> str:
    """Compile the library (always; a stale build is replaced atomically)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
