"""Build liblpc.so (the HIP library) in-tree with hipcc for gfx950.

    python -m fp8_precision_allreduce_amd.build

Flags: -O3; -ffp-contract=off so that every multiply and add in the
reductions is rounded on its own (the FP32 rank-order sum is defined that
way); packed FP32 instructions disabled in the device code generator.

Each source is compiled in two passes, as the HIP driver does internally:
the device pass (gfx950 code object bundle) and the host pass, which embeds
that bundle.  The packed-FP32 switch is a feature of the gfx950 code
generator, so it goes to the device pass only; the host objects are then
linked into the shared library.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblpc.so")
SOURCES = [os.path.join(CSRC, n) for n in ("lpc_kernels.hip", "lpc_api.hip", "lpc_allreduce.hip",
                                           "lpc_measure.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-ffp-contract=off",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]
DEVICE_ONLY = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd) -> None:
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.stdout.strip():
        print(p.stdout, file=sys.stderr, end="", flush=True)
    if p.returncode != 0:
        raise subprocess.CalledProcessError(p.returncode, cmd)


def _compile(src: str, work: str, verbose: bool) -> str:
    base = os.path.join(work, os.path.splitext(os.path.basename(src))[0])
    device = [HIPCC, *COMMON, *DEVICE_ONLY, "--cuda-device-only", "-o", base + ".hipfb", src]
    host = [HIPCC, *COMMON, "-fPIC", "--cuda-host-only", "-Xclang", "-fcuda-include-gpubinary",
            "-Xclang", base + ".hipfb", "-c", "-o", base + ".o", src]
    for cmd in (device, host):
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)
    return base + ".o"


def build(verbose: bool = False) -> str:
    """Compile every HIP source into liblpc.so (always recompiles); returns its path."""
    with tempfile.TemporaryDirectory(prefix="lpc_build_") as work:
        with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            objs = list(ex.map(lambda s: _compile(s, work, verbose), SOURCES))
        tmp = LIB + ".tmp%d" % os.getpid()
        link = [HIPCC, "--offload-arch=" + ARCH, "--hip-link", "-shared", "-fPIC", "-o", tmp, *objs]
        if verbose:
            print(" ".join(link), flush=True)
        _run(link)
        os.replace(tmp, LIB)
    return LIB


def assembly(out_dir: str) -> list:
    """Write the gfx950 assembly of each source to out_dir (for inspection)."""
    os.makedirs(out_dir, exist_ok=True)
    outs = []
    for src in SOURCES:
        out = os.path.join(out_dir, os.path.basename(src) + ".s")
        _run([HIPCC, *COMMON, *DEVICE_ONLY, "-S", "--cuda-device-only", "-o", out, src])
        outs.append(out)
    return outs


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
