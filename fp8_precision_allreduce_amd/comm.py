"""Torchcomms-shaped allreduce over N emulated ranks on one GPU.

The pages' quick-start creates a communicator, fills a tensor on every rank
and calls ``allreduce(t, ReduceOp.SUM, async_op=False)``: in place, on the
current stream, leaving the elementwise sum on every rank.  Their
low-precision collectives are switched on with the environment variable
``RCCL_LOW_PRECISION_ENABLE=1`` (infolabhq pages, low-precision section;
RCCLX post, quick-start section).  This module keeps that shape for a single
GPU: one communicator object stands for all N ranks, ``allreduce`` takes the
N ranks' tensors and reduces them in place through the library's
``lpc_allreduce_emulated`` (argument marshalling and padding only).

Padding: the low-precision algorithm needs n to be a multiple of 128*N and
DDA tree a multiple of 8*N.  A forced algorithm on a ragged size, and a
ragged fp32 size for which the library selects none, run on zero-padded
copies and write the real elements back; zeros change no sum and no block's
absmax.
"""
from __future__ import annotations

import os

import torch

from . import lpc


class ReduceOp:
    SUM = "sum"


def low_precision_from_env() -> bool:
    return os.environ.get("RCCL_LOW_PRECISION_ENABLE", "0").strip() not in ("", "0")


class EmulatedComm:
    """N ranks on one device.  rank r's data is the r-th tensor passed to a collective."""

    def __init__(self, nranks: int, device, name: str = "lpc", low_precision: bool | None = None):
        if not 1 <= nranks <= lpc.MAX_RANKS:
            raise ValueError("nranks must be in 1..%d (single node)" % lpc.MAX_RANKS)
        self.nranks = nranks
        self.device = torch.device(device)
        self.name = name
        self.low_precision = low_precision_from_env() if low_precision is None else bool(low_precision)

    def get_size(self) -> int:
        return self.nranks

    def get_device(self):
        return self.device

    def select_algo(self, n: int, dtype) -> int:
        return lpc.lpc_select_algo(self.nranks, n, dtype, self.low_precision)

    def allreduce(self, tensors, op=ReduceOp.SUM, async_op: bool = False, algo: int | None = None):
        """In-place SUM of the ranks' tensors; returns the algorithm used.  Work is
        enqueued on the current stream; async_op=False also waits for it."""
        if op != ReduceOp.SUM:
            raise ValueError("only ReduceOp.SUM is supported")
        if len(tensors) != self.nranks:
            raise ValueError("expected %d tensors, one per rank" % self.nranks)
        t0 = tensors[0]
        for t in tensors:
            if t.shape != t0.shape or t.dtype != t0.dtype or t.device != self.device or not t.is_contiguous():
                raise ValueError("rank tensors must be contiguous, on %s, of one shape and dtype" % self.device)
        n = t0.numel()
        if algo is None:
            algo = self.select_algo(n, t0.dtype)
            if algo == lpc.ALGO_AUTO and t0.dtype == torch.float32:
                algo = lpc.ALGO_DDA_TREE          # ragged fp32: tree on a zero-padded copy
        if algo == lpc.ALGO_AUTO:
            raise ValueError("no allreduce algorithm applies to %d elements of %s" % (n, t0.dtype))
        unit = {lpc.ALGO_LOW_PRECISION: lpc.BLOCK * self.nranks, lpc.ALGO_DDA_TREE: 8 * self.nranks}.get(algo, 1)
        padded = -(-n // unit) * unit if n else 0
        if padded != n:
            work = [torch.zeros(padded, dtype=t.dtype, device=self.device) for t in tensors]
            for w, t in zip(work, tensors):
                w[:n].copy_(t.reshape(-1))
        else:
            work = [t.reshape(-1) for t in tensors]
        ws = torch.empty(lpc.lpc_allreduce_workspace_bytes(algo, self.nranks, padded, t0.dtype),
                         dtype=torch.uint8, device=self.device)
        lpc.lpc_allreduce_emulated(work, algo, ws)
        if padded != n:
            for w, t in zip(work, tensors):
                t.reshape(-1).copy_(w[:n])
        if not async_op:
            torch.cuda.current_stream(self.device).synchronize()
        return algo


def new_comm(backend: str, device, name: str = "lpc", nranks: int = 8, low_precision: bool | None = None):
    """Communicator over `nranks` emulated ranks on `device` (backend name kept for the API's shape)."""
    return EmulatedComm(nranks, device, name, low_precision)
