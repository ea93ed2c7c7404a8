"""Build liblpc.so (the HIP library) in-tree with hipcc for gfx950.

    python -m fp8_precision_allreduce_amd.build

Flags: -O3; -ffp-contract=off so that every multiply and add in the
reductions is rounded on its own (the FP32 rank-order sum is defined that
way); packed FP32 instructions disabled in the device code generator.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblpc.so")
SOURCES = [os.path.join(CSRC, n) for n in ("lpc_kernels.hip", "lpc_api.hip", "lpc_allreduce.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into liblpc.so (always recompiles); returns its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


def assembly(out_dir: str) -> list:
    """Write the gfx950 assembly of each source to out_dir (for inspection)."""
    os.makedirs(out_dir, exist_ok=True)
    outs = []
    for src in SOURCES:
        out = os.path.join(out_dir, os.path.basename(src) + ".s")
        subprocess.check_call([HIPCC, *[f for f in FLAGS if f not in ("-shared",)], "-S",
                               "--cuda-device-only", "-o", out, src])
        outs.append(out)
    return outs


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
