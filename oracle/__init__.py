"""CPU oracle for the FP8 low-precision collective path (test infrastructure).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product library never imports
this package, and this package never imports the product library.

The arithmetic lives in ``lpc_oracle.c`` (plain single-threaded C, IEEE
binary32, no contraction).  This module compiles it with gcc, loads it with
ctypes and offers numpy-level wrappers.  Nothing here computes any step of the
method itself: it only marshals arrays.

bfloat16 arrays are carried as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lpc_oracle.c")
_LIB = os.path.join(_HERE, "liblpc_oracle.so")
_CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared"]
BLOCK = 128

_lock = threading.Lock()
_default = None


def build(force: bool = False, src: str = _SRC, lib: str = _LIB) -> str:
    """Compile the oracle C source into a shared library (gcc); returns its path."""
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(src):
        tmp = lib + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, src, "-lm"])
        os.replace(tmp, lib)
    return lib


_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_int = ctypes.c_int
_SIGNATURES = {
    "lpo_e4m3_decode": (ctypes.c_float, [ctypes.c_uint8]),
    "lpo_e4m3_encode": (ctypes.c_uint8, [ctypes.c_float]),
    "lpo_bf16_rne": (ctypes.c_uint16, [ctypes.c_float]),
    "lpo_e4m3_decode_array": (None, [_vp, _sz, _vp]),
    "lpo_e4m3_encode_array": (None, [_vp, _sz, _vp]),
    "lpo_bf16_rne_array": (None, [_vp, _sz, _vp]),
    "lpo_quantize_f32": (_int, [_vp, _sz, _vp, _vp]),
    "lpo_quantize_bf16": (_int, [_vp, _sz, _vp, _vp]),
    "lpo_dequantize_f32": (_int, [_vp, _vp, _sz, _vp]),
    "lpo_dequantize_bf16": (_int, [_vp, _vp, _sz, _vp]),
    "lpo_reduce_scatter_chunk": (_int, [_vp, _vp, _int, _int, _sz, _vp, _vp]),
    "lpo_allgather_dequant": (_int, [_vp, _vp, _int, _sz, _vp, _int]),
    "lpo_reduce_scatter_out": (_int, [_vp, _vp, _int, _int, _sz, _vp, _int]),
    "lpo_dda_flat_bf16": (_int, [_vp, _int, _sz, _vp]),
    "lpo_dda_tree_rs": (_int, [_vp, _int, _int, _int, _sz, _vp]),
    "lpo_a2av_route": (_int, [_vp, _sz, _int, _vp, _vp, _vp]),
    "lpo_quantize_rows": (_int, [_vp, _int, _sz, _sz, _vp, _vp, _vp]),
}


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _ptr_array(arrs):
    return (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments" % what)


def _as(a, dtype):
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def bf16_to_f32(h) -> np.ndarray:
    """Exact widening of bfloat16 patterns (a bit shift, no arithmetic)."""
    return (_as(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


class Oracle:
    """numpy-level wrappers around one loaded copy of the C oracle."""

    def __init__(self, libpath: str):
        lib = ctypes.CDLL(libpath)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        self.lib = lib
        self.path = libpath

    # -- codec ----------------------------------------------------------------
    def e4m3_decode(self, codes) -> np.ndarray:
        c = _as(codes, np.uint8)
        out = np.empty(c.shape, np.float32)
        self.lib.lpo_e4m3_decode_array(_p(c), c.size, _p(out))
        return out

    def e4m3_encode(self, x) -> np.ndarray:
        v = _as(x, np.float32)
        out = np.empty(v.shape, np.uint8)
        self.lib.lpo_e4m3_encode_array(_p(v), v.size, _p(out))
        return out

    def bf16_rne(self, x) -> np.ndarray:
        v = _as(x, np.float32)
        out = np.empty(v.shape, np.uint16)
        self.lib.lpo_bf16_rne_array(_p(v), v.size, _p(out))
        return out

    bf16_to_f32 = staticmethod(bf16_to_f32)

    # -- blockwise quantization -------------------------------------------------
    def quantize(self, x, bf16: bool = False):
        """Blockwise FP8 quantization of a flat buffer -> (codes u8[n], scales f32[n/128])."""
        v = _as(x, np.uint16 if bf16 else np.float32).reshape(-1)
        n = v.size
        codes = np.empty(n, np.uint8)
        scales = np.empty(n // BLOCK, np.float32)
        f = self.lib.lpo_quantize_bf16 if bf16 else self.lib.lpo_quantize_f32
        _check(f(_p(v), n, _p(codes), _p(scales)), "quantize")
        return codes, scales

    def dequantize(self, codes, scales, bf16: bool = False) -> np.ndarray:
        c = _as(codes, np.uint8).reshape(-1)
        s = _as(scales, np.float32).reshape(-1)
        if s.size * BLOCK != c.size:
            raise ValueError("dequantize: need one scale per 128 codes")
        out = np.empty(c.size, np.uint16 if bf16 else np.float32)
        f = self.lib.lpo_dequantize_bf16 if bf16 else self.lib.lpo_dequantize_f32
        _check(f(_p(c), _p(s), c.size, _p(out)), "dequantize")
        return out

    # -- low-precision allreduce steps -------------------------------------------
    def reduce_scatter_chunk(self, codes_list, scales_list, rank: int):
        """Reduce-scatter step for the chunk owned by ``rank`` -> (chunk codes, chunk scales)."""
        codes_list = [_as(c, np.uint8).reshape(-1) for c in codes_list]
        scales_list = [_as(s, np.float32).reshape(-1) for s in scales_list]
        N = len(codes_list)
        n = codes_list[0].size
        C = n // N
        cc = np.empty(C, np.uint8)
        cs = np.empty(C // BLOCK, np.float32)
        _check(self.lib.lpo_reduce_scatter_chunk(_ptr_array(codes_list), _ptr_array(scales_list),
                                                 N, rank, n, _p(cc), _p(cs)), "reduce_scatter_chunk")
        return cc, cs

    def allgather_dequant(self, chunk_codes, chunk_scales, bf16: bool = False) -> np.ndarray:
        chunk_codes = [_as(c, np.uint8).reshape(-1) for c in chunk_codes]
        chunk_scales = [_as(s, np.float32).reshape(-1) for s in chunk_scales]
        N = len(chunk_codes)
        n = chunk_codes[0].size * N
        out = np.empty(n, np.uint16 if bf16 else np.float32)
        _check(self.lib.lpo_allgather_dequant(_ptr_array(chunk_codes), _ptr_array(chunk_scales),
                                              N, n, _p(out), int(bf16)), "allgather_dequant")
        return out

    def reduce_scatter_out(self, codes_list, scales_list, rank: int, bf16: bool = False):
        """Standalone low-precision reduce-scatter: FP32 sum of the owned chunk, not requantized."""
        codes_list = [_as(c, np.uint8).reshape(-1) for c in codes_list]
        scales_list = [_as(s, np.float32).reshape(-1) for s in scales_list]
        N = len(codes_list)
        n = codes_list[0].size
        out = np.empty(n // N, np.uint16 if bf16 else np.float32)
        _check(self.lib.lpo_reduce_scatter_out(_ptr_array(codes_list), _ptr_array(scales_list),
                                               N, rank, n, _p(out), int(bf16)), "reduce_scatter_out")
        return out

    def lp_allreduce(self, xs, bf16: bool = False) -> dict:
        """The whole low-precision allreduce over all N ranks, keeping every intermediate.

        Returns dict(codes, scales, chunk_codes, chunk_scales, out); ``out`` is
        the result every rank holds.
        """
        q = [self.quantize(x, bf16) for x in xs]
        codes = [c for c, _ in q]
        scales = [s for _, s in q]
        chunks = [self.reduce_scatter_chunk(codes, scales, r) for r in range(len(xs))]
        cc = [c for c, _ in chunks]
        cs = [s for _, s in chunks]
        out = self.allgather_dequant(cc, cs, bf16)
        return dict(codes=codes, scales=scales, chunk_codes=cc, chunk_scales=cs, out=out)

    # -- DDA ----------------------------------------------------------------------
    def dda_flat(self, bufs) -> np.ndarray:
        """DDA flat local reduce of N bfloat16 buffers (uint16 patterns) -> bf16."""
        bufs = [_as(b, np.uint16).reshape(-1) for b in bufs]
        n = bufs[0].size
        out = np.empty(n, np.uint16)
        _check(self.lib.lpo_dda_flat_bf16(_ptr_array(bufs), len(bufs), n, _p(out)), "dda_flat")
        return out

    def dda_tree_rs(self, bufs, rank: int, bf16: bool) -> np.ndarray:
        """Unquantized reduce-scatter of the chunk owned by ``rank`` (float or bf16 buffers)."""
        bufs = [_as(b, np.uint16 if bf16 else np.float32).reshape(-1) for b in bufs]
        N = len(bufs)
        n = bufs[0].size
        out = np.empty(n // N, np.uint16 if bf16 else np.float32)
        _check(self.lib.lpo_dda_tree_rs(_ptr_array(bufs), int(bf16), N, rank, n, _p(out)),
               "dda_tree_rs")
        return out

    # -- all-to-all-v ----------------------------------------------------------------
    def a2av_route(self, dest, nranks: int):
        d = _as(dest, np.int32).reshape(-1)
        counts = np.empty(nranks, np.int32)
        offsets = np.empty(nranks, np.int32)
        perm = np.empty(d.size, np.int32)
        _check(self.lib.lpo_a2av_route(_p(d), d.size, nranks, _p(counts), _p(offsets), _p(perm)),
               "a2av_route")
        return counts, offsets, perm

    def quantize_rows(self, x, perm, bf16: bool = False):
        """Gather rows in ``perm`` order and quantize each -> packed (codes, scales), 2-D."""
        v = _as(x, np.uint16 if bf16 else np.float32)
        rows, row_len = v.shape
        p = _as(perm, np.int32).reshape(-1)
        if p.size != rows:
            raise ValueError("quantize_rows: perm needs one entry per row")
        codes = np.empty((rows, row_len), np.uint8)
        scales = np.empty((rows, row_len // BLOCK), np.float32)
        _check(self.lib.lpo_quantize_rows(_p(v), int(bf16), rows, row_len, _p(p), _p(codes),
                                          _p(scales)), "quantize_rows")
        return codes, scales


def default() -> Oracle:
    """The oracle built from lpc_oracle.c in this directory (compiled on first use)."""
    global _default
    with _lock:
        if _default is None:
            _default = Oracle(build())
    return _default


def __getattr__(name):
    # module-level access to the default oracle's methods: oracle.quantize(...), etc.
    if name.startswith("_"):
        raise AttributeError(name)
    return getattr(default(), name)
