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
SOURCES = [os.path.join(CSRC, n) for n in ("lpc_kernels.hip", "lpc_api.hip", "lpc_allreduce.hip",
                                           "lpc_measure.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


# The packed-FP32 switch is a device-code-generator feature: hipcc hands it to
# the host compilation too, whose target does not know it and says so once per
# source.  That one message is dropped; everything else the compiler prints is
# passed on.
_HOST_FEATURE_NOTE = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"


def _run(cmd) -> None:
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if l.strip() != _HOST_FEATURE_NOTE)
    if out.strip():
        print(out, file=sys.stderr, flush=True)
    if p.returncode != 0:
        raise subprocess.CalledProcessError(p.returncode, cmd)


def build(verbose: bool = False) -> str:
    """Compile every HIP source into liblpc.so (always recompiles); returns its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    _run(cmd)
    os.replace(tmp, LIB)
    return LIB


def assembly(out_dir: str) -> list:
    """Write the gfx950 assembly of each source to out_dir (for inspection)."""
    os.makedirs(out_dir, exist_ok=True)
    outs = []
    for src in SOURCES:
        out = os.path.join(out_dir, os.path.basename(src) + ".s")
        _run([HIPCC, *[f for f in FLAGS if f not in ("-shared",)], "-S", "--cuda-device-only", "-o", out, src])
        outs.append(out)
    return outs


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
