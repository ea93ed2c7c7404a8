"""The measurement reference kernels (include/lpc_measure.h) on the GPU: the plain
streaming kernel writes exactly its destination range with the documented values and
nothing past it, for every load:store ratio it picks; the empty launch writes nothing."""
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


def _expected(src_words: np.ndarray, nr: int, nw: int) -> np.ndarray:
    """The stream kernel's output as uint32 words [nw, 4], computed on the host from the
    kernel's documented lane layout: lane g of L lanes loads 16-byte vectors g + k*L (k < KR,
    below nr), xors them into (g, 0, 0, 0), and stores the result with its last word xored
    with k at vectors g + k*L (k < KW, below nw)."""
    if nr >= nw:
        kr, kw = (4 if nw == 0 else min(4, (nr + nw // 2) // nw)), 1
    else:
        kr, kw = 1, (4 if nr == 0 else min(4, (nw + nr // 2) // nr))
    lanes = max(-(-nr // kr), -(-nw // kw))
    L = -(-lanes // 256) * 256
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
                                   (16 * 1000, 16 * 3000), (16 * 4096, 16), (0, 16 * 777), (16 * 513, 0)],
                         ids=["copy", "fused_mix", "quantize_mix", "ragged_1to3", "read_heavy", "write_only",
                              "read_only"])
def test_stream_writes_its_range(dev, rb, wb):
    say("measure stream read=%d write=%d" % (rb, wb))
    g = np.random.Generator(np.random.PCG64(rb + 7 * wb))
    src_h = g.integers(0, 2 ** 32, max(rb, 16) // 4, dtype=np.uint32)
    src = torch.from_numpy(src_h.view(np.int32)).to(dev)
    dst = torch.full(((wb + 2 * GUARD) // 4,), -1, dtype=torch.int32, device=dev)
    body = dst[GUARD // 4:(GUARD + wb) // 4]
    lpc.lpc_measure_stream(src if rb else None, rb, body if wb else None, wb)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint32)
    assert np.all(got[:GUARD // 4] == 0xFFFFFFFF) and np.all(got[(GUARD + wb) // 4:] == 0xFFFFFFFF), \
        "the stream kernel wrote outside its destination"
    if wb:
        exp = _expected(src_h[:rb // 4], rb // 16, wb // 16)
        assert np.array_equal(got[GUARD // 4:(GUARD + wb) // 4].reshape(-1, 4), exp)


def test_stream_rejects_bad_sizes(dev):
    a = torch.zeros(64, dtype=torch.int32, device=dev)
    with pytest.raises(lpc.LpcError) as e:
        lpc.lpc_measure_stream(a, 24, a, 16)
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
