"""Python binding of liblpc.so: one function per C entry point, same names.

Argument marshalling only: each function checks that the torch tensors it is
given are contiguous GPU tensors of the right type and large enough for the
element count it derives, turns them into device pointers, and calls the C
entry point on torch's current HIP stream (or the stream given).  Every step
of the computation runs in the library's HIP kernels; there is no fallback.
A non-LPC_OK status raises LpcError.

bfloat16 data is passed as torch.bfloat16 tensors.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblpc.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "lpc.h")
MEASURE_HEADER = os.path.join(os.path.dirname(_HERE), "include", "lpc_measure.h")

BLOCK = 128
MAX_RANKS = 8
MAX_ELEMS = 1 << 32
LPC_F32, LPC_BF16 = 0, 1
ALGO_AUTO, ALGO_DDA_FLAT, ALGO_DDA_TREE, ALGO_LOW_PRECISION = 0, 1, 2, 3
ALGO_NAMES = {ALGO_AUTO: "auto", ALGO_DDA_FLAT: "dda_flat", ALGO_DDA_TREE: "dda_tree",
              ALGO_LOW_PRECISION: "low_precision"}
STATUS = ["LPC_OK", "LPC_ERR_NULL", "LPC_ERR_SHAPE", "LPC_ERR_RANKS", "LPC_ERR_DTYPE",
          "LPC_ERR_ALIGN", "LPC_ERR_HIP", "LPC_ERR_SCRATCH"]
NOALLOC_SCRATCH_BYTES = 64 << 20


class LpcError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s failed: %s" % (fn, msg))
        self.status = status
        self.status_name = STATUS[status] if 0 <= status < len(STATUS) else str(status)


_vp, _sz, _int = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
_pp = ctypes.POINTER(ctypes.c_void_p)
SIGNATURES = {
    "lpc_quantize_fp8": [_vp, _int, _sz, _vp, _vp, _vp],
    "lpc_reduce_scatter_chunk": [_pp, _pp, _int, _int, _sz, _vp, _vp, _vp],
    "lpc_allgather_dequant": [_pp, _pp, _int, _sz, _vp, _int, _vp],
    "lpc_rs_ag_fused": [_pp, _pp, _int, _int, _sz, _vp, _vp, _pp, _pp, _vp, _int, _vp],
    "lpc_reduce_scatter": [_pp, _pp, _int, _int, _sz, _vp, _int, _vp],
    "dda_flat_reduce": [_pp, _int, _sz, _vp, _vp],
    "dda_tree_reduce_scatter": [_pp, _int, _int, _int, _sz, _vp, _vp],
    "dda_tree_allgather": [_pp, _int, _int, _sz, _vp, _vp],
    "lpc_a2av_route": [_vp, _sz, _int, _vp, _vp, _vp, _vp],
    "lpc_quantize_fp8_rows": [_vp, _int, _sz, _sz, _vp, _vp, _vp, _vp],
    "lpc_dequantize_fp8": [_vp, _vp, _sz, _vp, _int, _vp],
    "lpc_e4m3_encode": [_vp, _sz, _vp, _vp],
    "lpc_select_algo": [_int, _sz, _int, _int],
    "lpc_allreduce_workspace_bytes": [_int, _int, _sz, _int, ctypes.POINTER(ctypes.c_size_t)],
    "lpc_allreduce_emulated": [_pp, _int, _sz, _int, _int, _vp, _sz, _vp],
    "lpc_allreduce_emulated_noalloc": [_pp, _int, _sz, _int, _int, _vp],
    # reference kernels for measurement (include/lpc_measure.h)
    "lpc_measure_stream": [_vp, _sz, _vp, _sz, _int, _vp],
    "lpc_measure_empty": [ctypes.c_uint, ctypes.c_uint, ctypes.c_uint, _sz, _vp, _vp],
}

_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded liblpc.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    "liblpc.so is not built (%s); build it with "
                    "`python -m fp8_precision_allreduce_amd.build` -- there is no fallback path"
                    % LIB_PATH)
            L = ctypes.CDLL(LIB_PATH)
            for name, args in SIGNATURES.items():
                f = getattr(L, name)
                f.argtypes = args
                f.restype = ctypes.c_int
            L.lpc_status_string.argtypes = [ctypes.c_int]
            L.lpc_status_string.restype = ctypes.c_char_p
            L.lpc_abi_version.argtypes = []
            L.lpc_abi_version.restype = ctypes.c_int
            _lib = L
    return _lib


def header_functions(header: str = HEADER) -> list:
    """Names of the functions a header under include/ declares (lpc.h by default)."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def lpc_status_string(status: int) -> str:
    return lib().lpc_status_string(status).decode()


def lpc_abi_version() -> int:
    return lib().lpc_abi_version()


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _call(name: str, *args):
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise LpcError(name, st, lpc_status_string(st))


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t: torch.Tensor, what: str, dtypes=None, min_numel: int = 0) -> ctypes.c_void_p:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % what)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor" % what)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % what)
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (what, t.dtype, dtypes))
    if t.numel() < min_numel:
        raise ValueError("%s holds %d elements, needs %d" % (what, t.numel(), min_numel))
    return ctypes.c_void_p(t.data_ptr())


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return LPC_F32
    if t.dtype == torch.bfloat16:
        return LPC_BF16
    raise TypeError("expected float32 or bfloat16, got %s" % t.dtype)


def _ptrs(ts, what, dtypes, min_numel, skip=None):
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        if i == skip and t is None:
            arr[i] = None
            continue
        arr[i] = _dev(t, "%s[%d]" % (what, i), dtypes, min_numel).value
    return arr


_U8 = (torch.uint8,)
_F32 = (torch.float32,)
_FB = (torch.float32, torch.bfloat16)
_I32 = (torch.int32,)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def lpc_quantize_fp8(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, stream=None):
    n = x.numel()
    _call("lpc_quantize_fp8", _dev(x, "x", _FB), _dtype(x), n, _dev(codes, "codes", _U8, n),
          _dev(scales, "scales", _F32, n // BLOCK), _stream(stream))


def lpc_reduce_scatter_chunk(codes, scales, rank: int, chunk_codes, chunk_scales, n: int = None,
                             stream=None):
    N = len(codes)
    n = codes[0].numel() if n is None else n
    _call("lpc_reduce_scatter_chunk", _ptrs(codes, "codes", _U8, n),
          _ptrs(scales, "scales", _F32, n // BLOCK), N, rank, n,
          _dev(chunk_codes, "chunk_codes", _U8, n // max(N, 1)),
          _dev(chunk_scales, "chunk_scales", _F32, n // max(N, 1) // BLOCK), _stream(stream))


def lpc_allgather_dequant(chunk_codes, chunk_scales, out: torch.Tensor, stream=None):
    N = len(chunk_codes)
    n = out.numel()
    C = n // max(N, 1)
    _call("lpc_allgather_dequant", _ptrs(chunk_codes, "chunk_codes", _U8, C),
          _ptrs(chunk_scales, "chunk_scales", _F32, C // BLOCK), N, n, _dev(out, "out", _FB),
          _dtype(out), _stream(stream))


def lpc_rs_ag_fused(codes, scales, rank: int, chunk_codes, chunk_scales, peer_chunk_codes,
                    peer_chunk_scales, out: torch.Tensor, stream=None):
    N = len(codes)
    n = out.numel()
    C = n // max(N, 1)
    _call("lpc_rs_ag_fused", _ptrs(codes, "codes", _U8, n), _ptrs(scales, "scales", _F32, n // BLOCK),
          N, rank, n, _dev(chunk_codes, "chunk_codes", _U8, C),
          _dev(chunk_scales, "chunk_scales", _F32, C // BLOCK),
          _ptrs(peer_chunk_codes, "peer_chunk_codes", _U8, C, skip=rank),
          _ptrs(peer_chunk_scales, "peer_chunk_scales", _F32, C // BLOCK, skip=rank),
          _dev(out, "out", _FB), _dtype(out), _stream(stream))


def lpc_reduce_scatter(codes, scales, rank: int, out: torch.Tensor, n: int = None, stream=None):
    N = len(codes)
    n = codes[0].numel() if n is None else n
    _call("lpc_reduce_scatter", _ptrs(codes, "codes", _U8, n), _ptrs(scales, "scales", _F32, n // BLOCK),
          N, rank, n, _dev(out, "out", _FB, n // max(N, 1)), _dtype(out), _stream(stream))


def dda_flat_reduce(bufs, out: torch.Tensor, stream=None):
    n = out.numel()
    _call("dda_flat_reduce", _ptrs(bufs, "bufs", (torch.bfloat16,), n), len(bufs), n,
          _dev(out, "out", (torch.bfloat16,)), _stream(stream))


def dda_tree_reduce_scatter(bufs, rank: int, out: torch.Tensor, stream=None):
    N = len(bufs)
    n = bufs[0].numel()
    _call("dda_tree_reduce_scatter", _ptrs(bufs, "bufs", (out.dtype,), n), _dtype(out), N, rank, n,
          _dev(out, "out", _FB, n // max(N, 1)), _stream(stream))


def dda_tree_allgather(chunks, out: torch.Tensor, stream=None):
    N = len(chunks)
    n = out.numel()
    _call("dda_tree_allgather", _ptrs(chunks, "chunks", (out.dtype,), n // max(N, 1)), _dtype(out), N, n,
          _dev(out, "out", _FB), _stream(stream))


def lpc_a2av_route(dest: torch.Tensor, nranks: int, counts, offsets, perm, stream=None):
    rows = dest.numel()
    _call("lpc_a2av_route", _dev(dest, "dest", _I32), rows, nranks,
          _dev(counts, "counts", _I32, nranks), _dev(offsets, "offsets", _I32, nranks),
          _dev(perm, "perm", _I32, rows), _stream(stream))


def lpc_quantize_fp8_rows(x: torch.Tensor, perm: torch.Tensor, codes, scales, stream=None):
    if x.dim() != 2:
        raise ValueError("x must be 2-D (rows x row_len)")
    rows, row_len = x.shape
    _call("lpc_quantize_fp8_rows", _dev(x, "x", _FB), _dtype(x), rows, row_len,
          _dev(perm, "perm", _I32, rows), _dev(codes, "codes", _U8, rows * row_len),
          _dev(scales, "scales", _F32, rows * row_len // BLOCK), _stream(stream))


def lpc_dequantize_fp8(codes, scales, out: torch.Tensor, stream=None):
    n = out.numel()
    _call("lpc_dequantize_fp8", _dev(codes, "codes", _U8, n), _dev(scales, "scales", _F32, n // BLOCK),
          n, _dev(out, "out", _FB), _dtype(out), _stream(stream))


def lpc_select_algo(nranks: int, n: int, dtype, low_precision_enabled: bool) -> int:
    """Algorithm the library picks for an allreduce of n elements per rank (no GPU call)."""
    t = LPC_BF16 if dtype == torch.bfloat16 else LPC_F32 if dtype == torch.float32 else 99
    return lib().lpc_select_algo(nranks, n, t, 1 if low_precision_enabled else 0)


def lpc_allreduce_workspace_bytes(algo: int, nranks: int, n: int, dtype) -> int:
    out = ctypes.c_size_t(0)
    t = LPC_BF16 if dtype == torch.bfloat16 else LPC_F32 if dtype == torch.float32 else 99
    _call("lpc_allreduce_workspace_bytes", algo, nranks, n, t, ctypes.byref(out))
    return out.value


def lpc_allreduce_emulated(bufs, algo: int, workspace: torch.Tensor, stream=None):
    """In-place allreduce (SUM) of the N rank buffers `bufs` (same shape and dtype)."""
    N = len(bufs)
    n = bufs[0].numel()
    dt = bufs[0].dtype
    _call("lpc_allreduce_emulated", _ptrs(bufs, "bufs", (dt,), n), N, n, _dtype(bufs[0]), algo,
          _dev(workspace, "workspace", _U8), workspace.numel(), _stream(stream))


def lpc_allreduce_emulated_noalloc(bufs, algo: int, stream=None):
    """lpc_allreduce_emulated with the library's static scratch in place of a workspace
    (allocates nothing; calls that overlap on one GPU race on the scratch)."""
    N = len(bufs)
    n = bufs[0].numel()
    dt = bufs[0].dtype
    _call("lpc_allreduce_emulated_noalloc", _ptrs(bufs, "bufs", (dt,), n), N, n, _dtype(bufs[0]), algo,
          _stream(stream))


def lpc_measure_stream(src, read_bytes: int, dst, write_bytes: int, per_lane: int = 0, stream=None):
    """Plain streaming kernel (measurement reference): reads read_bytes of src, writes write_bytes
    of dst (with write_bytes == 0, dst is a never-written sink of at least 16 bytes); per_lane 0
    is one round of resident wavefronts, 1/2/4/8 that many vectors per lane."""
    if src is not None and src.numel() * src.element_size() < read_bytes:
        raise ValueError("src holds fewer than %d bytes" % read_bytes)
    if dst is not None and dst.numel() * dst.element_size() < max(write_bytes, 16 if read_bytes else 0):
        raise ValueError("dst holds fewer than %d bytes" % max(write_bytes, 16))
    _call("lpc_measure_stream", _dev(src, "src") if src is not None else None, read_bytes,
          _dev(dst, "dst") if dst is not None else None, write_bytes, per_lane, _stream(stream))


def lpc_measure_empty(grid_x: int, grid_y: int, threads: int, kernarg_bytes: int, sink, stream=None):
    """Empty launch of the given shape (measurement reference); sink is never written."""
    _call("lpc_measure_empty", grid_x, grid_y, threads, kernarg_bytes, _dev(sink, "sink", None, 1),
          _stream(stream))


def lpc_e4m3_encode(x: torch.Tensor, codes: torch.Tensor, stream=None):
    n = x.numel()
    _call("lpc_e4m3_encode", _dev(x, "x", _F32), n, _dev(codes, "codes", _U8, n), _stream(stream))
