"""Seeded synthetic inputs for the FP8 low-precision collective path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no quantization, no rounding rule, no reduction), so both
the GPU library's tests and the CPU oracle's tests can consume it.

Workloads (one emulated rank's buffer each; rank r of a workload uses seed
``seed(name, r)``, numpy PCG64):

  lp_n4_64k_f32         N=4, 65,536 fp32 per rank, N(0, 1)
  dda_flat_n8_bf16      N=8, bf16, hidden 8192 x tokens {1,4,16,32}, N(0, 0.5)
  lp_n8_16MiB_f32       N=8, 4,194,304 fp32 per rank, N(0, 1), then
                        round(0.001*M) distinct positions scaled x100
  lp_n8_256MiB_bf16     N=8, 134,217,728 bf16 per rank, Laplace(0, b=1e-3)
  a2av_16384x7168_bf16  16,384 rows x 7168 bf16, N(0, 1); each row's
                        destination among 8 ranks drawn i.i.d. with
                        P(d) proportional to (d+1)^-1.2 (Zipf 1.2)

bfloat16 buffers are made by drawing fp32 and keeping the upper 16 bits of
each pattern (truncation); they are returned as uint16 bit patterns on the
host.  The largest workloads also have device-side generators that use
a seeded torch generator on the GPU, for runs where host generation and the
host-to-device copy would dominate; those draw a different (but equally
seeded) stream from the host generators.
"""
from __future__ import annotations

import numpy as np

SEED_BASE = 20260224
HIDDEN = 8192
DDA_TOKENS = (1, 4, 16, 32)
A2AV_ROWS = 16384
A2AV_ROW_LEN = 7168
A2AV_RANKS = 8
ZIPF_S = 1.2

LP_SMALL = "lp_n4_64k_f32"
DDA_FLAT = "dda_flat_n8_bf16"
LP_16MIB = "lp_n8_16MiB_f32"
LP_256MIB_BF16 = "lp_n8_256MiB_bf16"
A2AV = "a2av_16384x7168_bf16"

# `stream` keeps the workloads' seeds apart; `dist` names the value recipe
WORKLOADS = {
    LP_SMALL: dict(stream=1, nranks=4, n=65536, dtype="f32", dist="normal", scale=1.0),
    DDA_FLAT: dict(stream=2, nranks=8, n=HIDDEN * 4, dtype="bf16", dist="normal", scale=0.5),
    LP_16MIB: dict(stream=3, nranks=8, n=4194304, dtype="f32", dist="normal_outliers", scale=1.0),
    LP_256MIB_BF16: dict(stream=4, nranks=8, n=134217728, dtype="bf16", dist="laplace", scale=1e-3),
    A2AV: dict(stream=5, nranks=8, n=A2AV_ROWS * A2AV_ROW_LEN, dtype="bf16", dist="normal", scale=1.0),
}


def seed(name: str, rank: int) -> int:
    return SEED_BASE + 1000 * WORKLOADS[name]["stream"] + rank


def rng(name: str, rank: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed(name, rank)))


def truncate_to_bf16(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of each fp32 pattern, as uint16 (input generation only)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def normal_f32(g: np.random.Generator, n: int, sigma: float) -> np.ndarray:
    return (g.standard_normal(n, dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def with_outliers(g: np.random.Generator, x: np.ndarray, frac: float = 0.001,
                  factor: float = 100.0) -> np.ndarray:
    """Scale round(frac*n) distinct, uniformly chosen positions by ``factor``."""
    k = int(round(frac * x.size))
    idx = g.choice(x.size, size=k, replace=False)
    x = x.copy()
    x[idx] *= np.float32(factor)
    return x


def laplace_f32(g: np.random.Generator, n: int, b: float) -> np.ndarray:
    return g.laplace(0.0, b, n).astype(np.float32)


def rank_buffer(name: str, rank: int, n: int | None = None) -> np.ndarray:
    """Host buffer of emulated rank ``rank`` of workload ``name`` (float32 or uint16 bf16).

    ``n`` overrides the element count (smaller test sizes drawn with the same
    recipe and seed).
    """
    w = WORKLOADS[name]
    n = w["n"] if n is None else n
    g = rng(name, rank)
    if w["dist"] == "normal":
        x = normal_f32(g, n, w["scale"])
    elif w["dist"] == "normal_outliers":
        x = with_outliers(g, normal_f32(g, n, w["scale"]))
    elif w["dist"] == "laplace":
        x = laplace_f32(g, n, w["scale"])
    else:
        raise KeyError(w["dist"])
    return truncate_to_bf16(x) if w["dtype"] == "bf16" else x


def dda_buffers(tokens: int, nranks: int = 8, hidden: int = HIDDEN) -> list:
    """DDA flat: N bf16 buffers of hidden x tokens elements."""
    return [truncate_to_bf16(normal_f32(rng(DDA_FLAT, r), hidden * tokens, 0.5)) for r in range(nranks)]


def zipf_destinations(rows: int = A2AV_ROWS, nranks: int = A2AV_RANKS, s: float = ZIPF_S) -> np.ndarray:
    """Destination rank of every row, i.i.d. with P(d) proportional to (d+1)^-s."""
    w = (np.arange(nranks, dtype=np.float64) + 1.0) ** (-s)
    g = rng(A2AV, 999)
    return g.choice(nranks, size=rows, p=w / w.sum()).astype(np.int32)


def a2av_rows(rows: int = A2AV_ROWS, row_len: int = A2AV_ROW_LEN) -> np.ndarray:
    """All-to-all-v rows: rows x row_len bf16 (uint16) matrix, N(0, 1)."""
    return rank_buffer(A2AV, 0, rows * row_len).reshape(rows, row_len)


def pages_example(nranks: int) -> list:
    """The quick-start tensor on the pages: a 10 x 20 float tensor filled with the rank."""
    return [np.full((10, 20), float(r), dtype=np.float32) for r in range(nranks)]


# -- device-side generation for the largest workloads ---------------------------

def device_rank_buffer(name: str, rank: int, device, n: int | None = None):
    """Seeded torch generator on ``device``; returns a torch tensor (float32, or
    bfloat16 made by bit truncation).  Used where host generation would
    dominate (the 16 MiB and larger workloads at full size)."""
    import torch

    w = WORKLOADS[name]
    n = w["n"] if n is None else n
    gen = torch.Generator(device=device)
    gen.manual_seed(seed(name, rank))
    if w["dist"] in ("normal", "normal_outliers"):
        x = torch.randn(n, generator=gen, device=device, dtype=torch.float32) * w["scale"]
        if w["dist"] == "normal_outliers":
            k = int(round(0.001 * n))
            idx = torch.randperm(n, generator=gen, device=device)[:k]
            x[idx] *= 100.0
    elif w["dist"] == "laplace":
        # Laplace(0, b): sign * b * Exp(1)
        e = torch.empty(n, device=device, dtype=torch.float32).exponential_(generator=gen)
        sgn = torch.randint(0, 2, (n,), generator=gen, device=device, dtype=torch.int8)
        x = e * w["scale"]
        x = torch.where(sgn.bool(), -x, x)
        del e, sgn
    else:
        raise KeyError(w["dist"])
    if w["dtype"] == "bf16":
        x = (x.view(torch.int32) >> 16).to(torch.int16).view(torch.bfloat16)
    return x
