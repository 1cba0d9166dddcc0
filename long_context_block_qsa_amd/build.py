"""Build the QSA HIP library for gfx950 in-tree (``libqsa.so`` next to this file).

    python -m long_context_block_qsa_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqsa.so")
SOURCES = ["qsa_kernels.hip", "qsa_dense.hip", "qsa_backward.hip", "qsa_api.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden",
    # keep fp32 arithmetic out of packed (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the attention rescales them with VALU
    # instructions, which cannot address AGPRs (every tile would copy them back and forth)
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-Wall", "-Wno-unused-result",
]


def build(verbose: bool = False) -> str:
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libqsa.so")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
