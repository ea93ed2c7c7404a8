"""Seeded synthetic inputs for the FP8 low-precision collective path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no quantization, no rounding rule, no reduction), so both
the GPU library's tests and the CPU oracle's tests can consume it.

Workloads (one emulated rank's buffer each; rank r of a run uses seed
``seed(cfg, r)``, numpy PCG64):

  1  lp_allreduce_n4_64k_f32    N=4, 65,536 fp32 per rank, N(0, 1)
  2  dda_flat_n8_bf16           N=8, bf16, hidden 8192 x tokens {1,4,16,32},
                                N(0, 0.5)
  3  lp_allreduce_n8_16MiB_f32  N=8, 4,194,304 fp32 per rank, N(0, 1), then
                                round(0.001*M) distinct positions scaled x100
  4  lp_allreduce_n8_256MiB_bf16  N=8, 134,217,728 bf16 per rank,
                                Laplace(0, b=1e-3)
  5  a2av_16384x7168_bf16       16,384 rows x 7168 bf16, N(0, 1); each row's
                                destination among 8 ranks drawn i.i.d. with
                                P(d) proportional to (d+1)^-1.2 (Zipf 1.2)

bfloat16 buffers are made by drawing fp32 and keeping the upper 16 bits of
each pattern (truncation); they are returned as uint16 bit patterns on the
host.  The largest workloads (4, 5) also have device-side generators that use
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

CONFIGS = {
    1: dict(name="lp_allreduce_n4_64k_f32", nranks=4, n=65536, dtype="f32"),
    2: dict(name="dda_flat_n8_bf16", nranks=8, n=HIDDEN * 4, dtype="bf16"),
    3: dict(name="lp_allreduce_n8_16MiB_f32", nranks=8, n=4194304, dtype="f32"),
    4: dict(name="lp_allreduce_n8_256MiB_bf16", nranks=8, n=134217728, dtype="bf16"),
    5: dict(name="a2av_16384x7168_bf16", nranks=8, n=A2AV_ROWS * A2AV_ROW_LEN, dtype="bf16"),
}


def seed(cfg: int, rank: int) -> int:
    return SEED_BASE + 1000 * cfg + rank


def rng(cfg: int, rank: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed(cfg, rank)))


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


def rank_buffer(cfg: int, rank: int, n: int | None = None) -> np.ndarray:
    """Host buffer of emulated rank ``rank`` for workload ``cfg`` (float32 or uint16 bf16).

    ``n`` overrides the element count (smaller test sizes drawn with the same
    recipe and seed).
    """
    c = CONFIGS[cfg]
    n = c["n"] if n is None else n
    g = rng(cfg, rank)
    if cfg == 1:
        return normal_f32(g, n, 1.0)
    if cfg == 2:
        return truncate_to_bf16(normal_f32(g, n, 0.5))
    if cfg == 3:
        return with_outliers(g, normal_f32(g, n, 1.0))
    if cfg == 4:
        return truncate_to_bf16(laplace_f32(g, n, 1e-3))
    if cfg == 5:
        return truncate_to_bf16(normal_f32(g, n, 1.0))
    raise KeyError(cfg)


def dda_buffers(tokens: int, nranks: int = 8, hidden: int = HIDDEN) -> list:
    """Workload 2: N bf16 buffers of hidden x tokens elements."""
    return [truncate_to_bf16(normal_f32(rng(2, r), hidden * tokens, 0.5)) for r in range(nranks)]


def zipf_destinations(rows: int = A2AV_ROWS, nranks: int = A2AV_RANKS, s: float = ZIPF_S,
                      cfg: int = 5) -> np.ndarray:
    """Destination rank of every row, i.i.d. with P(d) proportional to (d+1)^-s."""
    w = (np.arange(nranks, dtype=np.float64) + 1.0) ** (-s)
    g = rng(cfg, 999)
    return g.choice(nranks, size=rows, p=w / w.sum()).astype(np.int32)


def a2av_rows(rows: int = A2AV_ROWS, row_len: int = A2AV_ROW_LEN) -> np.ndarray:
    """Workload 5: rows x row_len bf16 (uint16) matrix, N(0, 1)."""
    return rank_buffer(5, 0, rows * row_len).reshape(rows, row_len)


def pages_example(nranks: int) -> list:
    """The quick-start tensor on the pages: a 10 x 20 float tensor filled with the rank."""
    return [np.full((10, 20), float(r), dtype=np.float32) for r in range(nranks)]


# -- device-side generation for the largest workloads ---------------------------

def device_rank_buffer(cfg: int, rank: int, device, n: int | None = None):
    """Seeded torch generator on ``device``; returns a torch tensor (float32, or
    bfloat16 made by bit truncation).  Used where host generation would
    dominate (workloads 3-5 at full size)."""
    import torch

    c = CONFIGS[cfg]
    n = c["n"] if n is None else n
    gen = torch.Generator(device=device)
    gen.manual_seed(seed(cfg, rank))
    if cfg in (1, 3, 5):
        x = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
        if cfg == 3:
            k = int(round(0.001 * n))
            idx = torch.randperm(n, generator=gen, device=device)[:k]
            x[idx] *= 100.0
    elif cfg == 2:
        x = torch.randn(n, generator=gen, device=device, dtype=torch.float32) * 0.5
    elif cfg == 4:
        # Laplace(0, b): sign * b * Exp(1)
        e = torch.empty(n, device=device, dtype=torch.float32).exponential_(generator=gen)
        sgn = torch.randint(0, 2, (n,), generator=gen, device=device, dtype=torch.int8)
        x = e * 1e-3
        x = torch.where(sgn.bool(), -x, x)
        del e, sgn
    else:
        raise KeyError(cfg)
    if c["dtype"] == "bf16":
        x = (x.view(torch.int32) >> 16).to(torch.int16).view(torch.bfloat16)
    return x
