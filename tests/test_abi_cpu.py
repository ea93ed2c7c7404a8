"""The C ABI on the host, no GPU needed: the library loads, exports every function
include/lpc.h declares, and rejects bad arguments with the documented status
before touching the HIP runtime.

The pointers used here are fake addresses (aligned or not); every call below
is one that validation must refuse, so nothing is ever dereferenced or
launched.
"""
import ctypes
import re

import pytest

from fp8_precision_allreduce_amd import lpc

OK, NULL, SHAPE, RANKS, DTYPE, ALIGN, HIP, SCRATCH = range(8)
A = 0x10000        # a fake 16-byte-aligned device address
B = 0x10008        # a fake misaligned one
F32, BF16 = 0, 1
MAX_ELEMS = lpc.MAX_ELEMS


@pytest.fixture(scope="module")
def L():
    import torch

    # Fake addresses must never reach a kernel; if a call here wrongly passed
    # validation on a machine with a GPU it would launch on them.  These
    # checks are for the GPU-less host only.
    if torch.cuda.device_count() > 0:
        pytest.skip("fake-pointer ABI checks run only where no GPU is visible")
    return lpc.lib()


def arr(*ptrs):
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


def test_header_limits_match_binding():
    text = open(lpc.HEADER).read()
    assert re.search(r"#define LPC_MAX_ELEMS \(\(size_t\)1 << (\d+)\)", text).group(1) == "32"
    # the lane-vector kernels take 4 or more elements per lane; HIP accepts at
    # most 2^31 - 1 lanes along one grid dimension (the word-wide DDA kernels
    # cap their grid instead)
    assert MAX_ELEMS // 4 < 2 ** 31


def test_exports_every_declared_function(L):
    import glob
    import os

    headers = sorted(glob.glob(os.path.join(os.path.dirname(lpc.HEADER), "*.h")))
    assert lpc.HEADER in headers and lpc.MEASURE_HEADER in headers
    names = set()
    for h in headers:
        names |= set(lpc.header_functions(h))
    assert len(names) >= 18
    for name in names:
        assert hasattr(L, name), name
    assert set(lpc.SIGNATURES) | {"lpc_status_string", "lpc_abi_version"} == names


def test_measure_errors(L):
    s, e = L.lpc_measure_stream, L.lpc_measure_empty
    assert s(A, 16, A, 16 * 3 + 8, 0, None) == SHAPE
    assert s(A, 20, A, 16, 0, None) == SHAPE
    for bad in (-1, 3, 5, 16):
        assert s(A, 16, A + 1024, 16, bad, None) == SHAPE
    assert s(None, 0, None, 0, 0, None) == OK
    assert s(None, 16, A, 16, 0, None) == NULL
    assert s(A, 16, None, 16, 0, None) == NULL
    assert s(A, 16, None, 0, 0, None) == NULL              # read only: dst is the sink
    assert s(B, 16, A, 16, 0, None) == ALIGN
    assert s(A, 16, B, 16, 0, None) == ALIGN
    for k in (0, 1, 2, 4, 8):
        assert s(A, 16, A + 1024, 32, k, None) == HIP      # passes the checks; no device
    assert e(0, 1, 64, 8, A, None) == SHAPE
    assert e(1, 0, 64, 8, A, None) == SHAPE
    assert e(1, 1, 0, 8, A, None) == SHAPE
    assert e(1, 1, 2048, 8, A, None) == SHAPE
    assert e(1, 1, 64, 513, A, None) == SHAPE
    assert e(1, 1, 64, 8, None, None) == NULL
    assert e(1, 1, 64, 8, B, None) == ALIGN
    assert e(4, 2, 256, 300, A, None) == HIP


def test_abi_version_matches_header(L):
    m = re.search(r"#define LPC_ABI_VERSION (\d+)", open(lpc.HEADER).read())
    assert lpc.lpc_abi_version() == int(m.group(1))


def test_status_strings(L):
    for i, name in enumerate(lpc.STATUS):
        assert lpc.lpc_status_string(i).startswith(name)
    assert "unknown" in lpc.lpc_status_string(99)


def test_quantize_errors(L):
    f = L.lpc_quantize_fp8
    assert f(A, 7, 128, A, A, None) == DTYPE
    assert f(A, F32, 0, None, None, None) == OK          # n == 0: no-op, no pointer needed
    assert f(None, F32, 128, A, A, None) == NULL
    assert f(A, F32, 128, None, A, None) == NULL
    assert f(A, F32, 128, A, None, None) == NULL
    assert f(B, F32, 128, A, A, None) == ALIGN
    assert f(A, BF16, 128, B, A, None) == ALIGN
    assert f(A, F32, 128, A, A + 4, None) == ALIGN
    assert f(A, F32, 100, A, A, None) == SHAPE
    assert f(A, F32, 129, A, A, None) == SHAPE
    assert f(A, F32, MAX_ELEMS + 128, A, A, None) == SHAPE


@pytest.mark.parametrize("name", ["lpc_reduce_scatter_chunk"])
def test_reduce_scatter_chunk_errors(L, name):
    f = getattr(L, name)
    c4, s4 = arr(A, A, A, A), arr(A, A, A, A)
    assert f(c4, s4, 0, 0, 512, A, A, None) == RANKS
    assert f(c4, s4, 9, 0, 512, A, A, None) == RANKS
    assert f(c4, s4, 4, 4, 512, A, A, None) == RANKS
    assert f(c4, s4, 4, -1, 512, A, A, None) == RANKS
    assert f(c4, s4, 4, 0, 0, None, None, None) == OK
    assert f(None, s4, 4, 0, 512, A, A, None) == NULL
    assert f(arr(A, A, None, A), s4, 4, 0, 512, A, A, None) == NULL
    assert f(c4, arr(A, None, A, A), 4, 0, 512, A, A, None) == NULL
    assert f(c4, s4, 4, 0, 512, None, A, None) == NULL
    assert f(arr(A, A, A, B), s4, 4, 0, 512, A, A, None) == ALIGN
    assert f(c4, s4, 4, 0, 512, A, B, None) == ALIGN
    assert f(c4, s4, 4, 0, 256, A, A, None) == SHAPE      # not a multiple of 128*N
    assert f(c4, s4, 4, 0, 640, A, A, None) == SHAPE


def test_reduce_scatter_errors(L):
    f = L.lpc_reduce_scatter
    c2, s2 = arr(A, A), arr(A, A)
    assert f(c2, s2, 2, 0, 256, A, 3, None) == DTYPE
    assert f(c2, s2, 2, 2, 256, A, F32, None) == RANKS
    assert f(c2, s2, 2, 0, 256, None, F32, None) == NULL
    assert f(c2, s2, 2, 0, 256, B, BF16, None) == ALIGN
    assert f(c2, s2, 2, 0, 384, A, F32, None) == SHAPE


def test_allgather_errors(L):
    f = L.lpc_allgather_dequant
    c2, s2 = arr(A, A), arr(A, A)
    assert f(c2, s2, 2, 256, A, 2, None) == DTYPE
    assert f(c2, s2, 0, 256, A, F32, None) == RANKS
    assert f(c2, s2, 2, 0, None, F32, None) == OK
    assert f(c2, arr(None, A), 2, 256, A, F32, None) == NULL
    assert f(c2, s2, 2, 256, B, F32, None) == ALIGN
    assert f(c2, s2, 2, 128, A, F32, None) == SHAPE


def test_fused_errors(L):
    f = L.lpc_rs_ag_fused
    c2, s2 = arr(A, A), arr(A, A)
    assert f(c2, s2, 2, 0, 256, A, A, c2, s2, A, 5, None) == DTYPE
    assert f(c2, s2, 2, 2, 256, A, A, c2, s2, A, F32, None) == RANKS
    # the peer arrays' own-rank entry may be NULL ...
    assert f(c2, s2, 2, 0, 384, A, A, arr(None, A), arr(None, A), A, F32, None) == SHAPE
    # ... but no other entry
    assert f(c2, s2, 2, 0, 256, A, A, arr(A, None), arr(A, A), A, F32, None) == NULL
    assert f(c2, s2, 2, 1, 256, A, A, arr(None, A), arr(A, A), A, F32, None) == NULL
    assert f(c2, s2, 2, 0, 256, A, A, arr(None, A), arr(None, A), None, F32, None) == NULL
    assert f(c2, s2, 2, 0, 256, A, A, arr(None, B), arr(None, A), A, F32, None) == ALIGN
    assert f(c2, s2, 2, 0, 256, A, B, arr(None, A), arr(None, A), A, F32, None) == ALIGN


def test_dda_errors(L):
    f = L.dda_flat_reduce
    assert f(arr(A, A), 0, 16, A, None) == RANKS
    assert f(arr(A, A), 2, 0, None, None) == OK
    assert f(arr(A, None), 2, 16, A, None) == NULL
    assert f(arr(A, B), 2, 16, A, None) == ALIGN
    assert f(arr(A, A), 2, MAX_ELEMS + 1, A, None) == SHAPE
    g = L.dda_tree_reduce_scatter
    assert g(arr(A, A), 9, 2, 0, 32, A, None) == DTYPE
    assert g(arr(A, A), F32, 2, 3, 32, A, None) == RANKS
    assert g(arr(A, A), F32, 2, 0, 24, A, None) == SHAPE
    h = L.dda_tree_allgather
    assert h(arr(A, A), BF16, 2, 32, None, None) == NULL
    assert h(arr(A, A), BF16, 2, 40, A, None) == SHAPE


def test_a2av_errors(L):
    f = L.lpc_a2av_route
    assert f(A, 16, 0, A, A, A, None) == RANKS
    assert f(A, 0, 8, None, None, None, None) == OK
    assert f(A, 16, 8, A, None, A, None) == NULL
    assert f(A, 16, 8, A, A, B, None) == ALIGN
    assert f(A, 1 << 31, 8, A, A, A, None) == SHAPE
    g = L.lpc_quantize_fp8_rows
    assert g(A, 4, 16, 128, A, A, A, None) == DTYPE
    assert g(A, BF16, 16, 0, A, A, A, None) == OK
    assert g(A, BF16, 16, 128, None, A, A, None) == NULL
    assert g(A, BF16, 16, 128, A, A, B, None) == ALIGN
    assert g(A, BF16, 16, 100, A, A, A, None) == SHAPE
    d = L.lpc_dequantize_fp8
    assert d(A, A, 128, A, 2, None) == DTYPE
    assert d(A, None, 128, A, F32, None) == NULL
    assert d(A, A, 128, B, F32, None) == ALIGN
    assert d(A, A, 130, A, F32, None) == SHAPE
    e = L.lpc_e4m3_encode
    assert e(None, 5, A, None) == NULL
    assert e(A, 5, B, None) == ALIGN


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    """No silent fallback: a missing liblpc.so is an error, not a CPU path."""
    monkeypatch.setattr(lpc, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(lpc, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        lpc.lib()



AUTO, FLAT, TREE, LP = range(4)


def test_select_algo(L):
    f = L.lpc_select_algo
    assert f(8, 8192, BF16, 0) == FLAT                      # 16 KiB decode message
    assert f(8, 262144, BF16, 1) == FLAT                    # 512 KiB: still flat
    assert f(8, 262144 + 64, BF16, 1) == TREE               # just above the flat limit
    assert f(8, 4194304, F32, 0) == TREE                    # 16 MiB, low precision off
    assert f(8, 4194304, F32, 1) == LP                      # 16 MiB, low precision on
    assert f(8, 4194304 - 1024, F32, 1) == TREE             # below 16 MiB
    assert f(8, 4194304 + 64, F32, 1) == TREE               # not a multiple of 128*N
    assert f(8, 200, F32, 1) == AUTO                        # ragged fp32: nothing applies as given
    assert f(8, 201, BF16, 0) == FLAT
    assert f(3, 3 * 128 * 16384, BF16, 1) == TREE           # 12.6 MB of bf16: below the 16 MiB floor
    assert f(3, 3 * 128 * 21846, BF16, 1) == LP             # 16.8 MB of bf16, a multiple of 128*3
    assert f(0, 128, F32, 0) == AUTO and f(9, 128, F32, 0) == AUTO and f(8, 128, 7, 0) == AUTO


def test_allreduce_workspace_bytes(L):
    out = ctypes.c_size_t(0)
    g = L.lpc_allreduce_workspace_bytes
    n = 4194304
    assert g(LP, 8, n, F32, ctypes.byref(out)) == OK
    C = n // 8
    assert out.value == 8 * (n + n // 32) + 8 * (C + C // 32)   # every region is a 256-byte multiple here
    assert g(TREE, 8, n, F32, ctypes.byref(out)) == OK and out.value == 8 * C * 4
    assert g(FLAT, 8, 8192, BF16, ctypes.byref(out)) == OK and out.value == 8 * 8192 * 2
    assert g(FLAT, 3, 100, BF16, ctypes.byref(out)) == OK and out.value == 3 * 256   # 200 B rounded up
    assert g(FLAT, 8, 8192, F32, ctypes.byref(out)) == DTYPE
    assert g(AUTO, 8, 8192, F32, ctypes.byref(out)) == DTYPE
    assert g(LP, 8, 128 * 7, F32, ctypes.byref(out)) == SHAPE
    assert g(TREE, 8, 60, F32, ctypes.byref(out)) == SHAPE
    assert g(TREE, 9, 64, F32, ctypes.byref(out)) == RANKS
    assert g(TREE, 8, 64, F32, None) == NULL


def test_allreduce_emulated_errors(L):
    f = L.lpc_allreduce_emulated
    n = 8 * 128 * 4
    bufs = arr(*([A] * 8))
    ws_need = ctypes.c_size_t(0)
    assert L.lpc_allreduce_workspace_bytes(LP, 8, n, F32, ctypes.byref(ws_need)) == OK
    assert f(bufs, 8, n, F32, AUTO, A, ws_need.value, None) == DTYPE
    assert f(bufs, 8, n, F32, FLAT, A, ws_need.value, None) == DTYPE
    assert f(bufs, 9, n, F32, LP, A, ws_need.value, None) == RANKS
    assert f(bufs, 8, n + 128, F32, LP, A, 1 << 30, None) == SHAPE
    assert f(bufs, 8, 0, F32, LP, None, 0, None) == OK          # n == 0: no-op
    assert f(None, 8, n, F32, LP, A, ws_need.value, None) == NULL
    assert f(arr(*([A] * 7 + [None])), 8, n, F32, LP, A, ws_need.value, None) == NULL
    assert f(bufs, 8, n, F32, LP, None, ws_need.value, None) == NULL
    assert f(arr(*([A] * 7 + [B])), 8, n, F32, LP, A, ws_need.value, None) == ALIGN
    assert f(bufs, 8, n, F32, LP, B, ws_need.value, None) == ALIGN
    assert f(bufs, 8, n, F32, LP, A, ws_need.value - 1, None) == SHAPE


def test_allreduce_emulated_noalloc_errors(L):
    """The no-allocation variant checks what lpc_allreduce_emulated checks (no workspace
    arguments), then its static scratch's size; with no GPU visible a call that passes
    every check fails at the device lookup with LPC_ERR_HIP."""
    f = L.lpc_allreduce_emulated_noalloc
    n = 8 * 128 * 4
    bufs = arr(*([A] * 8))
    assert f(bufs, 8, n, F32, AUTO, None) == DTYPE
    assert f(bufs, 8, n, F32, FLAT, None) == DTYPE
    assert f(bufs, 9, n, F32, LP, None) == RANKS
    assert f(bufs, 8, n + 128, F32, LP, None) == SHAPE
    assert f(bufs, 8, 0, F32, LP, None) == OK                    # n == 0: no-op
    assert f(None, 8, n, F32, LP, None) == NULL
    assert f(arr(*([A] * 7 + [None])), 8, n, F32, LP, None) == NULL
    assert f(arr(*([A] * 7 + [B])), 8, n, F32, LP, None) == ALIGN
    big = 8 * 128 * 8192                                          # about 75 MiB of low-precision workspace
    need = ctypes.c_size_t(0)
    assert L.lpc_allreduce_workspace_bytes(LP, 8, big, F32, ctypes.byref(need)) == OK
    assert need.value > lpc.NOALLOC_SCRATCH_BYTES
    assert f(bufs, 8, big, F32, LP, None) == SCRATCH
    assert L.lpc_allreduce_workspace_bytes(TREE, 8, 8 * 8 * 2 ** 18, F32, ctypes.byref(need)) == OK
    assert need.value <= lpc.NOALLOC_SCRATCH_BYTES
    assert f(bufs, 8, 8 * 8 * 2 ** 18, F32, TREE, None) == HIP     # passes the checks; no device
    assert f(bufs, 8, n, F32, LP, None) == HIP


def test_noalloc_scratch_size_matches_header():
    m = re.search(r"#define LPC_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(lpc.HEADER).read())
    assert int(m.group(1)) << int(m.group(2)) == lpc.NOALLOC_SCRATCH_BYTES


def test_low_precision_switch_from_env(monkeypatch):
    from fp8_precision_allreduce_amd import comm

    monkeypatch.delenv("RCCL_LOW_PRECISION_ENABLE", raising=False)
    assert comm.low_precision_from_env() is False
    monkeypatch.setenv("RCCL_LOW_PRECISION_ENABLE", "1")
    assert comm.low_precision_from_env() is True
    monkeypatch.setenv("RCCL_LOW_PRECISION_ENABLE", "0")
    assert comm.low_precision_from_env() is False
    c = comm.EmulatedComm(4, "cpu", low_precision=None)
    assert c.low_precision is False and c.get_size() == 4


def test_launch_failure_is_reported(L):
    """A call that passes validation reaches the launch; with no GPU visible the
    launch itself fails, and that failure comes back as LPC_ERR_HIP (the status
    of the launch, not of some earlier call)."""
    assert L.lpc_quantize_fp8(A, F32, 128, A, A, None) == HIP
    assert L.lpc_dequantize_fp8(A, A, 128, A, BF16, None) == HIP
    assert L.dda_flat_reduce(arr(A, A), 2, 16, A, None) == HIP
    assert L.lpc_a2av_route(A, 16, 8, A, A, A, None) == HIP
    # validation still wins over the launch
    assert L.lpc_quantize_fp8(A, F32, 100, A, A, None) == SHAPE
