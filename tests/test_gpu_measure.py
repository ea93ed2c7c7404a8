"""The measurement reference kernels (include/lpc_measure.h) on the GPU: the plain
streaming kernel writes exactly its destination range with the documented values and
nothing past it, for every load:store count it picks (and nothing at all when it only
reads); the empty launch writes nothing."""
import numpy as np
import pytest
import torch

from fp8_precision_allreduce_amd import lpc

pytestmark = pytest.mark.gpu
GUARD = 4096


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lpc.lib()
    return torch.device("cuda:0")


def say(*a):
    print("[case]", *a, flush=True)


def _layout(nr: int, nw: int, per_lane: int):
    """(lanes L, loads per lane KR, stores per lane KW) the stream kernel picks.  per_lane 0: one
    round of 2,048 workgroups of 256 lanes when that leaves at most 8 vectors per lane each way,
    fewer workgroups when there is less to move, more at 8 per lane beyond; per_lane K: the
    workgroups K vectors per lane need.  Per-lane counts rounded up to 1, 2, 4 or 8."""
    m = max(nr, nw)
    if per_lane:
        wgs = -(-m // (256 * per_lane))
    else:
        need = -(-m // 256)
        wgs = need if need <= 2048 else (2048 if m <= 2048 * 256 * 8 else -(-m // (256 * 8)))
    L = wgs * 256
    bucket = lambda k: 0 if k == 0 else 1 if k <= 1 else 2 if k <= 2 else 4 if k <= 4 else 8
    return L, bucket(-(-nr // L)), bucket(-(-nw // L))


def _expected(src_words: np.ndarray, nr: int, nw: int, per_lane: int) -> np.ndarray:
    """The stream kernel's output as uint32 words [nw, 4], computed on the host from the
    kernel's documented lane layout: lane g of L lanes loads 16-byte vectors g + k*L (k < KR,
    below nr), xors them into (g, 0, 0, 0), and stores the result with its last word xored
    with k at vectors g + k*L (k < KW, below nw)."""
    L, kr, kw = _layout(nr, nw, per_lane)
    v = np.zeros((L, 4), np.uint32)
    v[:, 0] = np.arange(L, dtype=np.uint32)
    src = src_words.reshape(-1, 4)
    for k in range(kr):
        idx = np.arange(L) + k * L
        ok = idx < nr
        v[ok] ^= src[idx[ok]]
    out = np.zeros((nw, 4), np.uint32)
    for k in range(kw):
        idx = np.arange(L) + k * L
        ok = idx < nw
        w = v[ok].copy()
        w[:, 3] ^= np.uint32(k)
        out[idx[ok]] = w
    return out


@pytest.mark.parametrize("rb,wb", [(1 << 20, 1 << 20), (8_110_080, 17_317_888), (16 << 20, 4_325_376),
                                   (16 * 1000, 16 * 3000), (16 * 4096, 16), (0, 16 * 777), (16 * 513, 0),
                                   (64 << 20, 16), (48 << 20, 40 << 20)],
                         ids=["copy", "fused_mix", "quantize_mix", "ragged_1to3", "read_heavy", "write_only",
                              "read_only", "read_64MiB_beyond_one_round", "copy_48_40MiB"])
@pytest.mark.parametrize("per_lane", [0, 1, 2, 4, 8])
def test_stream_writes_its_range(dev, rb, wb, per_lane):
    say("measure stream read=%d write=%d per_lane=%d" % (rb, wb, per_lane))
    g = np.random.Generator(np.random.PCG64(rb + 7 * wb))
    src_h = g.integers(0, 2 ** 32, max(rb, 16) // 4, dtype=np.uint32)
    src = torch.from_numpy(src_h.view(np.int32)).to(dev)
    dst = torch.full(((wb + 2 * GUARD) // 4,), -1, dtype=torch.int32, device=dev)
    body = dst[GUARD // 4:(GUARD + wb) // 4]
    # with nothing to write, dst is the never-written sink: the guard-filled words must stay
    lpc.lpc_measure_stream(src if rb else None, rb, body if wb else dst[GUARD // 4:GUARD // 4 + 4], wb, per_lane)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint32)
    assert np.all(got[:GUARD // 4] == 0xFFFFFFFF) and np.all(got[(GUARD + wb) // 4:] == 0xFFFFFFFF), \
        "the stream kernel wrote outside its destination (or into the read-only sink)"
    if wb:
        exp = _expected(src_h[:rb // 4], rb // 16, wb // 16, per_lane)
        assert np.array_equal(got[GUARD // 4:(GUARD + wb) // 4].reshape(-1, 4), exp)


def test_stream_rejects_bad_sizes(dev):
    a = torch.zeros(64, dtype=torch.int32, device=dev)
    with pytest.raises(lpc.LpcError) as e:
        lpc.lpc_measure_stream(a, 24, a, 16)
    assert e.value.status_name == "LPC_ERR_SHAPE"
    with pytest.raises(lpc.LpcError) as e:
        lpc.lpc_measure_stream(a, 16, a[16:], 16, 3)
    assert e.value.status_name == "LPC_ERR_SHAPE"


@pytest.mark.parametrize("gx,gy,threads,kb", [(1, 1, 64, 16), (512, 7, 256, 296), (1024, 1, 256, 32),
                                              (3, 5, 1024, 512), (7, 1, 33, 100)])
def test_empty_launch_writes_nothing(dev, gx, gy, threads, kb):
    say("measure empty %dx%d x %d lanes, %d argument bytes" % (gx, gy, threads, kb))
    sink = torch.full((64,), 12345, dtype=torch.int32, device=dev)
    for _ in range(3):
        lpc.lpc_measure_empty(gx, gy, threads, kb, sink)
    torch.cuda.synchronize()
    assert bool((sink == 12345).all())
