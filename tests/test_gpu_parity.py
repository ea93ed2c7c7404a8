"""GPU parity: every HIP entry point against the CPU oracle, bit for bit.

The bar is byte equality everywhere (codes, scales, FP32 and bf16 outputs,
routing): both sides round every multiply and add separately in IEEE binary32
(no contraction), divide with a correctly rounded division, and use the same
E4M3 and bf16 round-to-nearest-even rules, so there is exactly one correct
result.  All calls go through the C ABI (ctypes binding); inputs are the
seeded generators' buffers.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_precision_allreduce_amd import inputs
from fp8_precision_allreduce_amd import lpc

pytestmark = pytest.mark.gpu
BLOCK = 128


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lpc.lib()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def say(*a):
    print("[case]", *a, flush=True)


# -- host <-> device helpers --------------------------------------------------

def to_dev(a: np.ndarray, dev) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def f32bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def assert_same(gpu: np.ndarray, ref: np.ndarray, what: str):
    if gpu.dtype == np.float32:
        gpu, ref = f32bits(gpu), f32bits(ref)
    bad = np.nonzero(gpu.reshape(-1) != ref.reshape(-1))[0]
    assert bad.size == 0, "%s: %d mismatches, first at %s: gpu %s ref %s" % (
        what, bad.size, bad[:4], gpu.reshape(-1)[bad[:4]], ref.reshape(-1)[bad[:4]])


def gpu_quantize(x_dev):
    n = x_dev.numel()
    codes = torch.empty(n, dtype=torch.uint8, device=x_dev.device)
    scales = torch.empty(n // BLOCK, dtype=torch.float32, device=x_dev.device)
    lpc.lpc_quantize_fp8(x_dev, codes, scales)
    return codes, scales


def gpu_lp_allreduce(xs_dev, out_dtype, fused=True):
    """All N ranks' steps on one GPU: quantize every rank, RS every chunk, then each
    rank's all-gather (fused kernel for the fused path)."""
    N = len(xs_dev)
    n = xs_dev[0].numel()
    C = n // N
    dev = xs_dev[0].device
    q = [gpu_quantize(x) for x in xs_dev]
    codes = [c for c, _ in q]
    scales = [s for _, s in q]
    cc = [torch.empty(C, dtype=torch.uint8, device=dev) for _ in range(N)]
    cs = [torch.empty(C // BLOCK, dtype=torch.float32, device=dev) for _ in range(N)]
    for r in range(N):
        lpc.lpc_reduce_scatter_chunk(codes, scales, r, cc[r], cs[r])
    outs = []
    for r in range(N):
        out = torch.empty(n, dtype=out_dtype, device=dev)
        if fused:
            own_c = torch.empty(C, dtype=torch.uint8, device=dev)
            own_s = torch.empty(C // BLOCK, dtype=torch.float32, device=dev)
            peers_c = [None if p == r else cc[p] for p in range(N)]
            peers_s = [None if p == r else cs[p] for p in range(N)]
            lpc.lpc_rs_ag_fused(codes, scales, r, own_c, own_s, peers_c, peers_s, out)
            assert torch.equal(own_c, cc[r]) and torch.equal(own_s.view(torch.int32), cs[r].view(torch.int32))
        else:
            lpc.lpc_allgather_dequant(cc, cs, out)
        outs.append(out)
    torch.cuda.synchronize()
    return dict(codes=codes, scales=scales, chunk_codes=cc, chunk_scales=cs, outs=outs)


def compare_allreduce(res, ref, what):
    N = len(res["codes"])
    for r in range(N):
        assert_same(to_host(res["codes"][r]), ref["codes"][r], "%s codes[%d]" % (what, r))
        assert_same(to_host(res["scales"][r]), ref["scales"][r], "%s scales[%d]" % (what, r))
        assert_same(to_host(res["chunk_codes"][r]), ref["chunk_codes"][r], "%s chunk codes[%d]" % (what, r))
        assert_same(to_host(res["chunk_scales"][r]), ref["chunk_scales"][r], "%s chunk scales[%d]" % (what, r))
    for r in range(N):
        assert_same(to_host(res["outs"][r]), ref["out"], "%s out on rank %d" % (what, r))


# -- codec ----------------------------------------------------------------------

def _codec_values():
    table = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float32)
    mids = ((table[:-1].astype(np.float64) + table[1:]) / 2).astype(np.float32)
    base = np.concatenate([table, mids, np.float32([464.0, 480.0, 500.0, 1e6, 3.4e38, 2.0 ** -10,
                                                     2.0 ** -11, 1e-40, 1.4e-45, 2.0 ** -126])])
    vals = [base]
    for k in range(1, 9):
        vals.append((f32bits(base) + np.uint32(k)).view(np.float32))
        vals.append((f32bits(base[base > 0]) - np.uint32(k)).view(np.float32))
    g = np.random.Generator(np.random.PCG64(101))
    rnd = g.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32).view(np.float32)
    vals.append(rnd[np.isfinite(rnd)])
    vals.append(g.uniform(-470, 470, 1 << 20).astype(np.float32))
    v = np.concatenate(vals).astype(np.float32)
    v = v[np.isfinite(v)]
    return np.concatenate([v, -v, np.float32([0.0, -0.0])])


def test_e4m3_encode_matches_oracle(dev, orc):
    v = _codec_values()
    say("e4m3 encode, %d values (+ragged tail)" % v.size)
    for n in (v.size, 7, 1):
        codes = torch.empty(n, dtype=torch.uint8, device=dev)
        lpc.lpc_e4m3_encode(to_dev(v[:n], dev), codes)
        assert_same(to_host(codes), orc.e4m3_encode(v[:n]), "encode n=%d" % n)


@pytest.mark.parametrize("lo_exp,hi_exp", [(-12, -5), (-5, 1), (1, 7), (7, 10)])
def test_e4m3_encode_every_float_in_binades(dev, orc, lo_exp, hi_exp):
    """Every float32 pattern with exponent in [lo, hi), both signs: together the ranges
    cover [2^-12, 2^10) in full -- everything below rounds to a signed zero, everything
    above saturates -- so every E4M3 rounding decision of the conversion instruction,
    subnormal, normal, tie and saturation, is compared with the oracle."""
    lo = np.uint32(f32bits(np.float32([2.0 ** lo_exp]))[0])
    hi = np.uint32(f32bits(np.float32([2.0 ** hi_exp]))[0])
    v = np.arange(lo, hi, dtype=np.uint32).view(np.float32)
    say("e4m3 encode every float in [2^%d, 2^%d): %d values" % (lo_exp, hi_exp, v.size))
    codes = torch.empty(v.size, dtype=torch.uint8, device=dev)
    xd = to_dev(v, dev)
    lpc.lpc_e4m3_encode(xd, codes)
    assert_same(to_host(codes), orc.e4m3_encode(v), "encode +")
    lpc.lpc_e4m3_encode(-xd, codes)
    assert_same(to_host(codes), orc.e4m3_encode(-v), "encode -")


# -- quantize / dequantize ---------------------------------------------------------------

def _edge_blocks():
    """Blocks that exercise the special cases: zeros of both signs, a scale that
    underflows, f32-denormal scales (saturating codes), one huge outlier, exact
    power-of-two values, a block of one repeated value."""
    g = np.random.Generator(np.random.PCG64(103))
    b = []
    b.append(np.zeros(BLOCK, np.float32))
    b.append(np.full(BLOCK, -0.0, np.float32))
    z = np.zeros(BLOCK, np.float32)
    z[7] = np.float32(1e-45)
    b.append(z)
    b.append((np.float32(2.0 ** -149) * g.integers(-700, 701, BLOCK)).astype(np.float32))
    b.append((np.float32(2.0 ** -140) * g.integers(-5, 6, BLOCK)).astype(np.float32))
    o = inputs.normal_f32(g, BLOCK, 1.0)
    o[3] = np.float32(1e30)
    b.append(o)
    b.append(np.ldexp(np.float32(1), g.integers(-30, 30, BLOCK)).astype(np.float32))
    b.append(np.full(BLOCK, np.float32(3.0), np.float32))
    b.append(inputs.normal_f32(g, BLOCK, 1e-30))
    b.append(inputs.normal_f32(g, BLOCK, 1e30))
    return np.concatenate(b)


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_quantize_matches_oracle(dev, orc, bf16):
    cases = {
        "lp_n4_64k_rank0": inputs.rank_buffer(inputs.LP_SMALL, 0),
        "ragged_37blocks": inputs.rank_buffer(inputs.LP_SMALL, 1, 37 * BLOCK),
        "one_block": inputs.rank_buffer(inputs.LP_SMALL, 2, BLOCK),
        "edge_blocks": _edge_blocks(),
        "lp_n8_16MiB_sample": inputs.rank_buffer(inputs.LP_16MIB, 0, 33 * 4096 + 5 * BLOCK),
    }
    for name, x in cases.items():
        if bf16:
            x = inputs.truncate_to_bf16(x)
        say("quantize", name, "bf16" if bf16 else "f32", x.size)
        codes, scales = gpu_quantize(to_dev(x, dev))
        rc, rs = orc.quantize(x, bf16=bf16)
        assert_same(to_host(codes), rc, name + " codes")
        assert_same(to_host(scales), rs, name + " scales")


def _bf16_blocks(amax_bits: int) -> np.ndarray:
    """Every finite bf16 value v with |v| <= amax (both signs), 127 to a block,
    each block led by amax itself so that all blocks share one scale."""
    pats = np.arange(1 << 16, dtype=np.uint32)
    vals = (pats << 16).view(np.float32)
    amax = np.float32((np.uint32(amax_bits) << 16).view(np.float32))
    keep = vals[np.isfinite(vals) & (np.abs(vals) <= amax)]
    pad = (-keep.size) % (BLOCK - 1)
    keep = np.concatenate([keep, np.zeros(pad, np.float32)]).reshape(-1, BLOCK - 1)
    return np.concatenate([np.full((keep.shape[0], 1), amax, np.float32), keep], axis=1).reshape(-1)


# block maxima: tiny; scales just below, at and just above 2^-80, the smallest
# scale the kernels' reciprocal quotient serves (amax = 1.75 * 2^-72 gives
# exactly 2^-80); ordinary; large; the largest finite bf16
_AMAX_BF16 = [0x0200, 0x1BDF, 0x1BE0, 0x1BE1, 0x1C40, 0x2A00, 0x3DCD, 0x3F80, 0x3FC0, 0x4040, 0x43E0,
              0x5F01, 0x7F7F]


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_quantize_every_bf16_value(dev, orc, bf16):
    """Every bf16 value under a range of block maxima, through the bf16 and the fp32
    input paths: bf16 quotients often fall exactly on E4M3 rounding midpoints."""
    x = np.concatenate([_bf16_blocks(a) for a in _AMAX_BF16])
    say("quantize every bf16 value", "bf16" if bf16 else "f32", x.size)
    xin = inputs.truncate_to_bf16(x) if bf16 else x
    codes, scales = gpu_quantize(to_dev(xin, dev))
    rc, rs = orc.quantize(xin, bf16=bf16)
    assert_same(to_host(scales), rs, "scales")
    assert_same(to_host(codes), rc, "codes")


def test_quantize_near_midpoints(dev, orc):
    """fp32 blocks whose quotients land on and within 12 ulps of E4M3 rounding
    midpoints, at scales from 2^-90 to 2^100 (both sides of 2^-80)."""
    g = np.random.Generator(np.random.PCG64(107))
    table = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = ((table[:-1] + table[1:]) / 2).astype(np.float32)
    nblk = 4096
    exps = np.concatenate([g.integers(-90, 100, nblk - 512), g.integers(-83, -77, 512)])
    s = np.ldexp(1.0 + g.integers(0, 1 << 23, nblk) / float(1 << 23), exps).astype(np.float32)
    q = mids[g.integers(0, mids.size, (nblk, BLOCK))]
    q = (f32bits(q).astype(np.int64) + g.integers(-12, 13, (nblk, BLOCK))).astype(np.uint32).view(np.float32)
    q = np.where(g.random((nblk, BLOCK)) < 0.5, -q, q)
    x = (q.astype(np.float64) * s[:, None]).astype(np.float32)
    x[:, 0] = (np.float64(448.0) * s).astype(np.float32)
    x = x.reshape(-1)
    say("quantize near midpoints", x.size)
    codes, scales = gpu_quantize(to_dev(x, dev))
    rc, rs = orc.quantize(x)
    assert_same(to_host(scales), rs, "scales")
    assert_same(to_host(codes), rc, "codes")


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_dequantize_matches_oracle(dev, orc, bf16):
    x = np.concatenate([inputs.rank_buffer(inputs.LP_SMALL, 3, 41 * BLOCK), _edge_blocks()])
    c, s = orc.quantize(x)
    say("dequantize", x.size, "bf16" if bf16 else "f32")
    out = torch.empty(x.size, dtype=torch.bfloat16 if bf16 else torch.float32, device=dev)
    lpc.lpc_dequantize_fp8(to_dev(c, dev), to_dev(s, dev), out)
    assert_same(to_host(out), orc.dequantize(c, s, bf16=bf16), "dequantize")


def test_zero_size_calls_are_noops(dev):
    say("n == 0 no-ops")
    e = torch.empty(0, device=dev)
    lpc.lpc_quantize_fp8(e, torch.empty(0, dtype=torch.uint8, device=dev), torch.empty(0, device=dev))
    lpc.dda_flat_reduce([torch.empty(0, dtype=torch.bfloat16, device=dev)] * 2,
                        torch.empty(0, dtype=torch.bfloat16, device=dev))
    torch.cuda.synchronize()


# -- low-precision allreduce ---------------------------------------------------------------------

@pytest.mark.parametrize("fused", [True, False], ids=["fused", "unfused"])
def test_lp_allreduce_n4_64k(dev, orc, fused):
    N = inputs.WORKLOADS[inputs.LP_SMALL]["nranks"]
    xs = [inputs.rank_buffer(inputs.LP_SMALL, r) for r in range(N)]
    say("lp allreduce N=%d n=%d fused=%s" % (N, xs[0].size, fused))
    res = gpu_lp_allreduce([to_dev(x, dev) for x in xs], torch.float32, fused)
    compare_allreduce(res, orc.lp_allreduce(xs), "n4 64k")


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "unfused"])
def test_lp_allreduce_rank_counts(dev, orc, N, bf16, fused):
    """Every rank count 1..8 (one template instance each), ragged chunks (an odd
    number of blocks, so the last wavefront is half empty, and a workgroup count
    that is not a multiple of the 8 XCDs), both dtypes, fused and unfused."""
    n = BLOCK * N * 37
    xs = [inputs.rank_buffer(inputs.LP_16MIB, r, n) for r in range(N)]
    if bf16:
        xs = [inputs.truncate_to_bf16(x) for x in xs]
    say("lp allreduce N=%d n=%d bf16=%s fused=%s" % (N, n, bf16, fused))
    res = gpu_lp_allreduce([to_dev(x, dev) for x in xs], torch.bfloat16 if bf16 else torch.float32, fused)
    compare_allreduce(res, orc.lp_allreduce(xs, bf16=bf16), "N=%d" % N)


def _random_case(g):
    """Rank count, size, dtype and a mix of block magnitudes drawn from g: blocks
    scaled by 10^U(-30, 30), zero blocks, blocks with a single huge outlier."""
    N = int(g.integers(1, 9))
    blocks = int(g.integers(1, 48))
    n = BLOCK * N * blocks
    bf16 = bool(g.integers(0, 2))
    xs = []
    for _ in range(N):
        x = g.standard_normal(n).astype(np.float32).reshape(-1, BLOCK)
        x *= (10.0 ** g.uniform(-30, 30, (x.shape[0], 1))).astype(np.float32)
        x[g.random(x.shape[0]) < 0.05] = 0.0
        hot = g.random(x.shape[0]) < 0.05
        x[hot, g.integers(0, BLOCK)] *= np.float32(1e4)
        x = np.nan_to_num(x.reshape(-1), posinf=np.float32(3e38), neginf=np.float32(-3e38))
        xs.append(inputs.truncate_to_bf16(x) if bf16 else x)
    return N, n, bf16, xs


@pytest.mark.parametrize("seed", range(24))
def test_lp_allreduce_random_cases(dev, orc, seed):
    """Randomly drawn rank counts, sizes, dtypes and block magnitudes (seeded), both
    paths (fused on even seeds), every intermediate against the oracle."""
    g = np.random.Generator(np.random.PCG64(900 + seed))
    N, n, bf16, xs = _random_case(g)
    fused = seed % 2 == 0
    say("lp allreduce random seed=%d N=%d n=%d bf16=%s fused=%s" % (seed, N, n, bf16, fused))
    res = gpu_lp_allreduce([to_dev(x, dev) for x in xs], torch.bfloat16 if bf16 else torch.float32, fused)
    compare_allreduce(res, orc.lp_allreduce(xs, bf16=bf16), "random seed %d" % seed)


@pytest.mark.parametrize("chunk_blocks", [1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 63, 64, 65, 8 * 64 + 3])
@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_fused_chunk_sizes(dev, orc, chunk_blocks, bf16):
    """Chunk sizes around the wavefront (2 blocks of 4-wide lanes, 4 of 8-wide),
    workgroup (8 or 16 blocks) and XCD (8 workgroups) granularities: every tile of
    the XCD-aware order is visited exactly once, for both lane widths."""
    N = 8
    n = BLOCK * N * chunk_blocks
    xs = [inputs.rank_buffer(inputs.LP_SMALL, r, n) for r in range(N)]
    if bf16:
        xs = [inputs.truncate_to_bf16(x) for x in xs]
    say("fused chunk of %d blocks, N=8, bf16=%s" % (chunk_blocks, bf16))
    res = gpu_lp_allreduce([to_dev(x, dev) for x in xs], torch.bfloat16 if bf16 else torch.float32, True)
    compare_allreduce(res, orc.lp_allreduce(xs, bf16=bf16), "chunk_blocks=%d" % chunk_blocks)


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "unfused"])
@pytest.mark.parametrize("N,C", [(2, 2097408), (3, 1048832), (5, 524544), (8, 524416)],
                         ids=["N2", "N3", "N5", "N8-odd-blocks"])
def test_fused_grid_beyond_one_round(dev, orc, N, C, fused):
    """Chunks just past the size where one lane vector per lane would take more than
    one round of wavefronts (8,192): the fp32 fused and all-gather launches give each lane
    two vectors, half a chunk apart (N = 2, 3, 5); with an odd number of blocks per chunk
    (N = 8) they keep one.  Every rank's launches, every intermediate, in full."""
    n = C * N
    xs = [inputs.rank_buffer(inputs.LP_16MIB, r, n) for r in range(N)]
    say("beyond one round: N=%d C=%d n=%d fused=%s" % (N, C, n, fused))
    res = gpu_lp_allreduce([to_dev(x, dev) for x in xs], torch.float32, fused)
    compare_allreduce(res, orc.lp_allreduce(xs), "N=%d C=%d" % (N, C))


def test_quantize_and_dequantize_at_the_largest_size(dev, orc):
    """n = LPC_MAX_ELEMS (2^32 fp32 elements, 16 GiB): quantize and dequantize at
    the largest accepted size, where byte offsets pass 2^32 and the grid is at its
    widest.  Checked on blocks on both sides of every 1 GiB of input (so of every
    4 GiB byte boundary), the first and last block, and 64 random blocks."""
    n = lpc.MAX_ELEMS
    nblk = n // BLOCK
    say("quantize + dequantize at n = %d" % n)
    gen = torch.Generator(device=dev)
    gen.manual_seed(113)
    x = torch.randn(n, generator=gen, device=dev, dtype=torch.float32)
    codes, scales = gpu_quantize(x)
    back = torch.empty(n, dtype=torch.bfloat16, device=dev)
    lpc.lpc_dequantize_fp8(codes, scales, back)
    torch.cuda.synchronize()
    marks = [0, nblk - 1] + [k * (nblk // 16) + d for k in range(1, 16) for d in (-1, 0)]
    rng = np.random.Generator(np.random.PCG64(113))
    blocks = np.unique(np.concatenate([np.array(marks), rng.integers(0, nblk, 64)]))
    bidx = torch.from_numpy(blocks).to(dev)
    idx = (bidx[:, None] * BLOCK + torch.arange(BLOCK, device=dev)[None, :]).reshape(-1)
    xb = to_host(x[idx])
    rc, rs = orc.quantize(xb)
    assert_same(to_host(codes[idx]), rc, "max-size codes")
    assert_same(to_host(scales[bidx]), rs, "max-size scales")
    assert_same(to_host(back[idx]), orc.dequantize(rc, rs, bf16=True), "max-size dequantize")
    del x, codes, scales, back
    torch.cuda.empty_cache()


def test_fused_at_the_largest_size(dev, orc):
    """The fused RS+AG at n = LPC_MAX_ELEMS per rank with N = 8 (the last rank, so
    that the own chunk ends at element 2^32): every rank's quantized buffer, the
    reduce-scatter chunks and the fp32 output, checked on sampled blocks of every
    chunk, including each chunk's first and last block."""
    N = 8
    n = lpc.MAX_ELEMS
    C = n // N
    r = N - 1
    say("fused RS+AG at n = %d, N = %d, rank %d" % (n, N, r))
    gen = torch.Generator(device=dev)
    rng = np.random.Generator(np.random.PCG64(127))
    per_chunk = [np.unique(np.concatenate([[0, C // BLOCK - 1], rng.integers(0, C // BLOCK, 24)]))
                 for _ in range(N)]
    codes, scales, xb = [], [], []
    for s_ in range(N):
        gen.manual_seed(1000 + s_)
        x = torch.randn(n, generator=gen, device=dev, dtype=torch.float32)
        c, sc = gpu_quantize(x)
        codes.append(c)
        scales.append(sc)
        # inputs of the sampled blocks of every chunk, kept on the host
        xb.append([to_host(x[(torch.from_numpy(p * C // BLOCK + per_chunk[p]).to(dev)[:, None] * BLOCK +
                               torch.arange(BLOCK, device=dev)[None, :]).reshape(-1)]) for p in range(N)])
        del x
    cc = [torch.empty(C, dtype=torch.uint8, device=dev) for _ in range(N)]
    cs = [torch.empty(C // BLOCK, dtype=torch.float32, device=dev) for _ in range(N)]
    for p in range(N):
        if p != r:
            lpc.lpc_reduce_scatter_chunk(codes, scales, p, cc[p], cs[p])
    out = torch.empty(n, dtype=torch.float32, device=dev)
    lpc.lpc_rs_ag_fused(codes, scales, r, cc[r], cs[r], [None if p == r else cc[p] for p in range(N)],
                        [None if p == r else cs[p] for p in range(N)], out)
    torch.cuda.synchronize()
    for p in range(N):
        blocks = per_chunk[p]
        qb = [orc.quantize(xb[s_][p]) for s_ in range(N)]
        gidx = torch.from_numpy(((p * C // BLOCK + blocks)[:, None] * BLOCK + np.arange(BLOCK)[None, :])
                                .reshape(-1)).to(dev)
        for s_ in range(N):
            assert_same(to_host(codes[s_][gidx]), qb[s_][0], "max-size codes rank %d chunk %d" % (s_, p))
        sum_codes, sum_scales = orc.reduce_scatter_chunk([np.tile(c, N) for c, _ in qb],
                                                         [np.tile(sc, N) for _, sc in qb], 0)
        lidx = torch.from_numpy((blocks[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)).to(dev)
        assert_same(to_host(cc[p][lidx]), sum_codes, "max-size chunk codes %d" % p)
        assert_same(to_host(cs[p][torch.from_numpy(blocks).to(dev)]), sum_scales, "max-size chunk scales %d" % p)
        assert_same(to_host(out[gidx]), orc.dequantize(sum_codes, sum_scales), "max-size out chunk %d" % p)
    del codes, scales, cc, cs, out
    torch.cuda.empty_cache()


def test_graph_replays_match_eager(dev):
    """A caller may capture the step (quantize + fused RS+AG + DDA flat) in a HIP
    graph: replay it three times with eager work and synchronisation in between,
    and check every replay against the eager result."""
    N = 8
    n = BLOCK * N * 40
    C = n // N
    xs = [to_dev(inputs.rank_buffer(inputs.LP_16MIB, r, n), dev) for r in range(N)]
    q = [gpu_quantize(x) for x in xs]
    codes = [c for c, _ in q]
    scales = [s for _, s in q]
    cc = [torch.empty(C, dtype=torch.uint8, device=dev) for _ in range(N)]
    cs = [torch.empty(C // BLOCK, dtype=torch.float32, device=dev) for _ in range(N)]
    for r in range(N):
        lpc.lpc_reduce_scatter_chunk(codes, scales, r, cc[r], cs[r])
    bufs = [to_dev(b, dev) for b in inputs.dda_buffers(1)]
    own_c = torch.empty(C, dtype=torch.uint8, device=dev)
    own_s = torch.empty(C // BLOCK, dtype=torch.float32, device=dev)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    dout = torch.empty_like(bufs[0])
    q0c = torch.empty(n, dtype=torch.uint8, device=dev)
    q0s = torch.empty(n // BLOCK, dtype=torch.float32, device=dev)

    def step():
        lpc.lpc_quantize_fp8(xs[0], q0c, q0s)
        lpc.lpc_rs_ag_fused(codes, scales, 0, own_c, own_s, [None] + cc[1:], [None] + cs[1:], out)
        lpc.dda_flat_reduce(bufs, dout)

    say("graph replay vs eager")
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (q0c, q0s, own_c, own_s, out, dout)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (q0c, q0s, own_c, own_s, out, dout):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((q0c, q0s, own_c, own_s, out, dout), ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "replay %d differs" % rep


def test_graph_replays_match_eager_a2av(dev):
    """All-to-all-v route + row quantize + dequantize captured in one HIP graph:
    every replay reproduces the eager result (the router's multi-workgroup
    counting keeps no state between calls)."""
    rows, row_len = 5000, 1024
    x = to_dev(inputs.a2av_rows(rows, row_len), dev)
    dest = to_dev(inputs.zipf_destinations(rows=rows), dev)
    counts = torch.empty(8, dtype=torch.int32, device=dev)
    offsets = torch.empty(8, dtype=torch.int32, device=dev)
    perm = torch.empty(rows, dtype=torch.int32, device=dev)
    codes = torch.empty(rows * row_len, dtype=torch.uint8, device=dev)
    scales = torch.empty(rows * row_len // BLOCK, dtype=torch.float32, device=dev)
    back = torch.empty(rows, row_len, dtype=torch.bfloat16, device=dev)

    def step():
        lpc.lpc_a2av_route(dest, 8, counts, offsets, perm)
        lpc.lpc_quantize_fp8_rows(x, perm, codes, scales)
        lpc.lpc_dequantize_fp8(codes, scales, back)

    say("graph replay vs eager, all-to-all-v")
    outs = (counts, offsets, perm, codes, scales, back)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "replay %d differs" % rep


def test_lp_allreduce_pages_example(dev):
    """The Torchcomms quick-start on the pages: 10x20 tensors of the rank, SUM -> N(N-1)/2
    everywhere (padded with zeros to whole blocks per chunk)."""
    for N in (2, 4, 8):
        say("pages example N=%d" % N)
        xs = inputs.pages_example(N)
        n = xs[0].size
        unit = BLOCK * N
        padded = -(-n // unit) * unit
        bufs = [to_dev(np.concatenate([x.reshape(-1), np.zeros(padded - n, np.float32)]), dev) for x in xs]
        res = gpu_lp_allreduce(bufs, torch.float32)
        for out in res["outs"]:
            assert torch.all(out[:n] == N * (N - 1) / 2)


@pytest.fixture(scope="module")
def lp_16mib(orc):
    xs = [inputs.rank_buffer(inputs.LP_16MIB, r) for r in range(8)]
    return xs, orc.lp_allreduce(xs)


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "unfused"])
def test_lp_allreduce_n8_16MiB_full(dev, lp_16mib, fused):
    """The 16 MiB workload at full size (N=8, 16 MiB fp32 per rank, outliers), every intermediate,
    through the fused launch and through the reduce-scatter and all-gather launches."""
    xs, ref = lp_16mib
    say("lp allreduce 16 MiB full N=8 n=%d fused=%s" % (xs[0].size, fused))
    res = gpu_lp_allreduce([to_dev(x, dev) for x in xs], torch.float32, fused)
    compare_allreduce(res, ref, "n8 16MiB")


def test_lp_allreduce_n8_256MiB_bf16(dev, orc):
    """The 256 MiB bf16 workload at full size (N=8, 256 MiB bf16 per rank, Laplace): the whole path
    on the GPU (fused kernel for ranks 0 and 7).  The last chunk (rank 7's, at the highest
    offsets of every buffer: 16,777,216 elements) is compared in full: every rank's codes and
    scales over it, the requantized chunk, and both fused launches' bf16 output over it (rank
    7's from registers, rank 0's from the peer chunk).  The other chunks are compared on 96
    sampled blocks each, first and last block included."""
    N = 8
    n = inputs.WORKLOADS[inputs.LP_256MIB_BF16]["n"]
    C = n // N
    say("lp allreduce 256 MiB bf16 full-size N=8 n=%d (sampled check)" % n)
    xs = [inputs.device_rank_buffer(inputs.LP_256MIB_BF16, r, dev) for r in range(N)]
    q = [gpu_quantize(x) for x in xs]
    codes = [c for c, _ in q]
    scales = [s for _, s in q]
    cc = [torch.empty(C, dtype=torch.uint8, device=dev) for _ in range(N)]
    cs = [torch.empty(C // BLOCK, dtype=torch.float32, device=dev) for _ in range(N)]
    for r in range(N):
        lpc.lpc_reduce_scatter_chunk(codes, scales, r, cc[r], cs[r])
    g = np.random.Generator(np.random.PCG64(107))
    outs = []
    for r in (0, N - 1):
        out = torch.empty(n, dtype=torch.bfloat16, device=dev)
        own_c = torch.empty(C, dtype=torch.uint8, device=dev)
        own_s = torch.empty(C // BLOCK, dtype=torch.float32, device=dev)
        lpc.lpc_rs_ag_fused(codes, scales, r, own_c, own_s, [None if p == r else cc[p] for p in range(N)],
                            [None if p == r else cs[p] for p in range(N)], out)
        torch.cuda.synchronize()
        assert torch.equal(own_c, cc[r]) and torch.equal(own_s.view(torch.int32), cs[r].view(torch.int32))
        for p in range(N):
            blocks = np.sort(g.choice(C // BLOCK, size=96, replace=False))
            blocks[0], blocks[-1] = 0, C // BLOCK - 1          # first and last block of the chunk
            idx = torch.from_numpy(((p * C // BLOCK + blocks)[:, None] * BLOCK +
                                    np.arange(BLOCK)[None, :]).reshape(-1)).to(dev)
            xb = [to_host(x[idx]) for x in xs]                   # inputs of those blocks, every rank
            for s_ in range(N):
                rc, rs = orc.quantize(xb[s_], bf16=True)
                assert_same(to_host(codes[s_][idx]), rc, "256 MiB codes rank %d" % s_)
                assert_same(to_host(scales[s_][torch.from_numpy(p * C // BLOCK + blocks).to(dev)]), rs,
                            "256 MiB scales rank %d" % s_)
            # the sampled blocks form a little allreduce of their own (block-local arithmetic)
            qb = [orc.quantize(x, bf16=True) for x in xb]
            m = blocks.size * BLOCK
            sum_codes, sum_scales = orc.reduce_scatter_chunk([np.tile(c, N) for c, _ in qb],
                                                             [np.tile(s, N) for _, s in qb], 0)
            assert sum_codes.size == m
            lidx = torch.from_numpy((blocks[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)).to(dev)
            assert_same(to_host(cc[p][lidx]), sum_codes, "256 MiB chunk codes %d" % p)
            assert_same(to_host(cs[p][torch.from_numpy(blocks).to(dev)]), sum_scales, "256 MiB chunk scales %d" % p)
            ref_out = orc.dequantize(sum_codes, sum_scales, bf16=True)
            assert_same(to_host(out[idx]), ref_out, "256 MiB out rank %d chunk %d" % (r, p))
        outs.append(out)
    # the last chunk in full: the oracle over that chunk of every rank's buffer
    p = N - 1
    sl, slb = slice(p * C, (p + 1) * C), slice(p * C // BLOCK, (p + 1) * C // BLOCK)
    say("lp allreduce 256 MiB bf16: chunk %d in full (%d elements per rank)" % (p, C))
    qc = []
    for s_ in range(N):
        rc, rs = orc.quantize(to_host(xs[s_][sl]), bf16=True)
        assert_same(to_host(codes[s_][sl]), rc, "256 MiB chunk %d codes rank %d (full)" % (p, s_))
        assert_same(to_host(scales[s_][slb]), rs, "256 MiB chunk %d scales rank %d (full)" % (p, s_))
        full_c = np.zeros(n, np.uint8)
        full_s = np.zeros(n // BLOCK, np.float32)
        full_c[sl], full_s[slb] = rc, rs
        qc.append((full_c, full_s))
    sum_codes, sum_scales = orc.reduce_scatter_chunk([c for c, _ in qc], [s_ for _, s_ in qc], p)
    del qc
    assert_same(to_host(cc[p]), sum_codes, "256 MiB chunk %d requantized codes (full)" % p)
    assert_same(to_host(cs[p]), sum_scales, "256 MiB chunk %d requantized scales (full)" % p)
    ref_out = orc.dequantize(sum_codes, sum_scales, bf16=True)
    for r, out in zip((0, N - 1), outs):
        assert_same(to_host(out[sl]), ref_out, "256 MiB out rank %d chunk %d (full)" % (r, p))
    del xs, codes, scales, cc, cs, outs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_lp_reduce_scatter_one_quantization(dev, orc, bf16):
    """Low-precision ReduceScatter: the FP32 rank-order sum of the owned chunk, unquantized."""
    N = 8
    n = BLOCK * N * 19
    xs = [inputs.rank_buffer(inputs.LP_16MIB, r, n) for r in range(N)]
    q = [orc.quantize(x) for x in xs]
    codes = [to_dev(c, dev) for c, _ in q]
    scales = [to_dev(s, dev) for _, s in q]
    for r in (0, 3, N - 1):
        say("lp reduce-scatter rank %d bf16=%s" % (r, bf16))
        out = torch.empty(n // N, dtype=torch.bfloat16 if bf16 else torch.float32, device=dev)
        lpc.lpc_reduce_scatter(codes, scales, r, out)
        ref = orc.reduce_scatter_out([c for c, _ in q], [s for _, s in q], r, bf16=bf16)
        assert_same(to_host(out), ref, "reduce_scatter rank %d" % r)


# -- DDA ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("tokens", inputs.DDA_TOKENS)
def test_dda_flat_message_sizes(dev, orc, tokens):
    bufs = inputs.dda_buffers(tokens)
    say("dda flat N=8 hidden 8192 x %d tokens" % tokens)
    out = torch.empty(bufs[0].size, dtype=torch.bfloat16, device=dev)
    lpc.dda_flat_reduce([to_dev(b, dev) for b in bufs], out)
    assert_same(to_host(out), orc.dda_flat(bufs), "dda flat T=%d" % tokens)


@pytest.mark.parametrize("N,n", [(1, 8), (2, 3), (4, 1), (8, 2), (2, 4), (3, 1001), (8, 8 * 977 + 5),
                                 (5, 4096 * 3 + 7), (8, 64 * 4 + 3)])
def test_dda_flat_ragged(dev, orc, N, n):
    """Even and odd element counts (an odd last element goes to a launch of its own), a single
    element (the tail launch alone), and nothing written past n."""
    bufs = [inputs.truncate_to_bf16(inputs.normal_f32(inputs.rng(inputs.DDA_FLAT, r), n, 0.5)) for r in range(N)]
    say("dda flat ragged N=%d n=%d" % (N, n))
    guard = torch.full((n + 64,), -7.0, dtype=torch.bfloat16, device=dev)
    out = guard[:n]
    lpc.dda_flat_reduce([to_dev(b, dev) for b in bufs], out)
    assert_same(to_host(out), orc.dda_flat(bufs), "dda flat ragged")
    assert bool((guard[n:] == -7.0).all()), "dda flat wrote past n"


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
@pytest.mark.parametrize("N,n", [(1, 8 * 37), (2, 2 * 8 * 5), (8, 8 * 8), (3, 3 * 8 * 77), (5, 5 * 8 * 1001)])
def test_dda_tree_rs_guarded(dev, orc, bf16, N, n):
    """One rank's tree reduce-scatter at chunk sizes that leave a partial workgroup, for the
    first and the last rank, and nothing written past the chunk."""
    fb = [inputs.normal_f32(inputs.rng(inputs.DDA_FLAT, r), n, 0.5) for r in range(N)]
    bufs = [inputs.truncate_to_bf16(x) for x in fb] if bf16 else fb
    dt = torch.bfloat16 if bf16 else torch.float32
    bd = [to_dev(b, dev) for b in bufs]
    C = n // N
    for r in (0, N - 1):
        say("dda tree rs guarded N=%d n=%d rank %d bf16=%s" % (N, n, r, bf16))
        guard = torch.full((C + 64,), -7.0, dtype=dt, device=dev)
        lpc.dda_tree_reduce_scatter(bd, r, guard[:C])
        assert_same(to_host(guard[:C]), orc.dda_tree_rs(bufs, r, bf16), "dda tree rs %d" % r)
        assert bool((guard[C:] == -7.0).all()), "dda tree rs wrote past the chunk"


@pytest.mark.parametrize("what", ["tree_rs_f32", "tree_rs_bf16", "flat_bf16"])
def test_dda_word_kernels_at_the_largest_size(dev, what):
    """One rank of n = LPC_MAX_ELEMS: 2^32 or 2^31 words, more than one launch has lanes for,
    so the grid stops short and its lanes take every grid-size-th word.  With one rank the
    reduce is the identity (bf16 -> fp32 -> bf16 is exact); checked on words on both sides of
    every 1/16 of the buffer, the first and last ones and 4,096 random ones."""
    n = lpc.MAX_ELEMS
    dt = torch.float32 if what == "tree_rs_f32" else torch.bfloat16
    say("%s at n = %d, N = 1" % (what, n))
    gen = torch.Generator(device=dev)
    gen.manual_seed(117)
    x = torch.randn(n, generator=gen, device=dev, dtype=torch.float32).to(dt)
    out = torch.zeros(n, dtype=dt, device=dev)
    if what == "flat_bf16":
        lpc.dda_flat_reduce([x], out)
    else:
        lpc.dda_tree_reduce_scatter([x], 0, out)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(117))
    marks = [0, 1, n - 2, n - 1] + [k * (n // 16) + d for k in range(1, 16) for d in (-1, 0)]
    idx = torch.from_numpy(np.unique(np.concatenate([np.array(marks), rng.integers(0, n, 4096)]))).to(dev)
    iv = torch.int32 if dt == torch.float32 else torch.int16
    assert torch.equal(out[idx].view(iv), x[idx].view(iv)), "max-size %s" % what
    del x, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_dda_tree(dev, orc, bf16):
    N, n = 8, 8 * 8 * 1001
    fb = [inputs.normal_f32(inputs.rng(inputs.DDA_FLAT, r), n, 0.5) for r in range(N)]
    bufs = [inputs.truncate_to_bf16(x) for x in fb] if bf16 else fb
    dt = torch.bfloat16 if bf16 else torch.float32
    bd = [to_dev(b, dev) for b in bufs]
    chunks = []
    for r in range(N):
        say("dda tree rs rank %d bf16=%s" % (r, bf16))
        out = torch.empty(n // N, dtype=dt, device=dev)
        lpc.dda_tree_reduce_scatter(bd, r, out)
        assert_same(to_host(out), orc.dda_tree_rs(bufs, r, bf16), "dda tree rs %d" % r)
        chunks.append(out)
    full = torch.empty(n, dtype=dt, device=dev)
    lpc.dda_tree_allgather(chunks, full)
    assert_same(to_host(full), np.concatenate([to_host(c) for c in chunks]), "dda tree allgather")
    if bf16:
        assert_same(to_host(full), orc.dda_flat(bufs), "dda tree == dda flat")


# -- all-to-all-v ----------------------------------------------------------------------------------

def test_a2av_route_sizes(dev, orc):
    # one workgroup per sub-tile (1024 rows, 2048 from 18,432 rows) up to 128
    # workgroups, then larger tiles: sizes around a sub-tile, ragged tails,
    # multi-sub-tile tiles, whole counting rounds (16 x 1024 and 8 x 2048
    # rows) with and without a partial round, and both sides of the switch
    for rows, nranks in ((inputs.A2AV_ROWS, 8), (1, 8), (1000, 3), (1023, 8), (1024, 8), (1025, 5),
                         (4097, 1), (16_383, 8), (16_384, 6), (16_385, 8), (17_408, 8), (18_431, 8), (18_432, 8),
                         (32_768, 4), (34_817, 8), (70_000, 8), (140_000, 7), (300_001, 8)):
        dest = inputs.zipf_destinations(rows=rows, nranks=nranks)
        say("a2av route rows=%d nranks=%d" % (rows, nranks))
        counts = torch.empty(nranks, dtype=torch.int32, device=dev)
        offsets = torch.empty(nranks, dtype=torch.int32, device=dev)
        perm = torch.empty(rows, dtype=torch.int32, device=dev)
        lpc.lpc_a2av_route(to_dev(dest, dev), nranks, counts, offsets, perm)
        rc, ro, rp = orc.a2av_route(dest, nranks)
        assert_same(to_host(counts), rc, "counts")
        assert_same(to_host(offsets), ro, "offsets")
        assert_same(to_host(perm), rp, "perm")


def test_a2av_route_drops_bad_destinations(dev):
    dest = np.array([3, 9, 0, -1, 7, 0], np.int32)
    say("a2av route with out-of-range destinations")
    counts = torch.empty(8, dtype=torch.int32, device=dev)
    offsets = torch.empty(8, dtype=torch.int32, device=dev)
    perm = torch.empty(6, dtype=torch.int32, device=dev)
    lpc.lpc_a2av_route(to_dev(dest, dev), 8, counts, offsets, perm)
    assert to_host(counts).tolist() == [2, 0, 0, 1, 0, 0, 0, 1]
    assert to_host(offsets).tolist() == [0, 2, 2, 2, 3, 3, 3, 3]
    assert to_host(perm).tolist() == [2, 5, 0, 4, -1, -1]


def test_a2av_route_drops_bad_destinations_large(dev, orc):
    """Out-of-range destinations spread over many workgroups: the valid rows are
    routed as the oracle routes them alone, and perm's tail is -1."""
    rng = np.random.default_rng(11)
    # bad values: negative, at or past 8, and (with fewer than 8 ranks) in nranks..7,
    # spread over whole counting rounds and partial ones
    for rows, bad, nranks in ((5000, 0.15, 8), (140_000, 0.02, 8), (3000, 1.0, 8), (40_000, 0.05, 5),
                              (20_000, 0.3, 3), (16_384, 0.1, 7), (70_001, 0.01, 2)):
        dest = inputs.zipf_destinations(rows=rows, nranks=nranks).copy()
        hit = rng.random(rows) < bad
        pool = np.array([-1, -7, 8, 9, 12, 2 ** 31 - 1] + list(range(nranks, 8)), np.int64)
        dest[hit] = pool[rng.integers(0, pool.size, int(hit.sum()))].astype(np.int32)
        say("a2av route rows=%d nranks=%d with %d out-of-range destinations" % (rows, nranks, int(hit.sum())))
        counts = torch.empty(nranks, dtype=torch.int32, device=dev)
        offsets = torch.empty(nranks, dtype=torch.int32, device=dev)
        perm = torch.empty(rows, dtype=torch.int32, device=dev)
        lpc.lpc_a2av_route(to_dev(dest, dev), nranks, counts, offsets, perm)
        keep = np.nonzero(~hit)[0].astype(np.int32)
        rc, ro, rp = (orc.a2av_route(dest[keep], nranks) if keep.size
                      else (np.zeros(nranks, np.int32),) * 2 + (keep,))
        want = np.full(rows, -1, np.int32)
        want[:keep.size] = keep[rp]
        assert_same(to_host(counts), rc, "counts")
        assert_same(to_host(offsets), ro, "offsets")
        assert_same(to_host(perm), want, "perm")


def test_a2av_quantize_rows_small(dev, orc):
    rows, row_len = 300, inputs.A2AV_ROW_LEN
    x = inputs.a2av_rows(rows, row_len)
    _, _, perm = orc.a2av_route(inputs.zipf_destinations(rows=rows), 8)
    perm_bad = perm.copy()
    perm_bad[5] = -1
    perm_bad[9] = rows
    for name, p in (("routed", perm), ("with invalid entries", perm_bad)):
        say("a2av quantize rows", name)
        codes = torch.empty((rows, row_len), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, row_len // BLOCK), dtype=torch.float32, device=dev)
        lpc.lpc_quantize_fp8_rows(to_dev(x, dev), to_dev(p, dev), codes, scales)
        if name == "routed":
            rc, rs = orc.quantize_rows(x, p, bf16=True)
        else:
            rc, rs = orc.quantize_rows(x, perm, bf16=True)
            for k in (5, 9):
                rc[k] = 0
                rs[k] = 0.0
        assert_same(to_host(codes), rc, "rows codes")
        assert_same(to_host(scales), rs, "rows scales")
    # long rows (16,640 elements, 130 blocks): a row spans many workgroups' granule tiles, and tiles
    # start and end inside rows
    x2 = inputs.truncate_to_bf16(inputs.normal_f32(inputs.rng(inputs.A2AV, 1), 6 * 128 * 130, 1.0)).reshape(6, -1)
    p2 = np.array([5, 0, 3, 1, 4, 2], np.int32)
    say("a2av quantize long rows", x2.shape)
    codes = torch.empty(x2.shape, dtype=torch.uint8, device=dev)
    scales = torch.empty((6, x2.shape[1] // BLOCK), dtype=torch.float32, device=dev)
    lpc.lpc_quantize_fp8_rows(to_dev(x2, dev), to_dev(p2, dev), codes, scales)
    rc, rs = orc.quantize_rows(x2, p2, bf16=True)
    assert_same(to_host(codes), rc, "long rows codes")
    assert_same(to_host(scales), rs, "long rows scales")


def test_a2av_16384x7168(dev, orc):
    """The all-to-all-v workload at full size: route, quantize + pack all 16,384 x 7168 rows, dequantize
    the packed buffer; the permutation, every packed row's codes and scales and the whole
    dequantized buffer compared with the oracle."""
    rows, row_len = inputs.A2AV_ROWS, inputs.A2AV_ROW_LEN
    say("a2av full rows=%d row_len=%d" % (rows, row_len))
    x = inputs.a2av_rows()
    dest = inputs.zipf_destinations()
    xd, dd = to_dev(x, dev), to_dev(dest, dev)
    counts = torch.empty(8, dtype=torch.int32, device=dev)
    offsets = torch.empty(8, dtype=torch.int32, device=dev)
    perm = torch.empty(rows, dtype=torch.int32, device=dev)
    lpc.lpc_a2av_route(dd, 8, counts, offsets, perm)
    codes = torch.empty((rows, row_len), dtype=torch.uint8, device=dev)
    scales = torch.empty((rows, row_len // BLOCK), dtype=torch.float32, device=dev)
    lpc.lpc_quantize_fp8_rows(xd, perm, codes, scales)
    back = torch.empty((rows, row_len), dtype=torch.bfloat16, device=dev)
    lpc.lpc_dequantize_fp8(codes, scales, back)
    torch.cuda.synchronize()
    rc, ro, rp = orc.a2av_route(dest, 8)
    assert_same(to_host(perm), rp, "a2av perm")
    assert_same(to_host(counts), rc, "a2av counts")
    assert_same(to_host(offsets), ro, "a2av offsets")
    assert int(to_host(counts).sum()) == rows
    say("a2av full: oracle quantize + dequantize of all %d rows" % rows)
    qc, qs = orc.quantize_rows(x, rp, bf16=True)
    assert_same(to_host(codes), qc.reshape(rows, row_len), "a2av packed codes (all rows)")
    assert_same(to_host(scales), qs.reshape(rows, row_len // BLOCK), "a2av packed scales (all rows)")
    ref_back = orc.dequantize(qc.reshape(-1), qs.reshape(-1), bf16=True)
    assert_same(to_host(back).reshape(-1), ref_back, "a2av dequantized rows (all)")


# -- emulated allreduce (size-based dispatch, torchcomms-shaped wrapper) ------------------------------

def _oracle_allreduce(orc, xs, algo, bf16):
    N = len(xs)
    if algo == lpc.ALGO_DDA_FLAT:
        return orc.dda_flat(xs)
    if algo == lpc.ALGO_DDA_TREE:
        return np.concatenate([orc.dda_tree_rs(xs, r, bf16) for r in range(N)])
    return orc.lp_allreduce(xs, bf16=bf16)["out"]


@pytest.mark.parametrize("algo,bf16", [(lpc.ALGO_DDA_FLAT, True), (lpc.ALGO_DDA_TREE, False),
                                       (lpc.ALGO_DDA_TREE, True), (lpc.ALGO_LOW_PRECISION, False),
                                       (lpc.ALGO_LOW_PRECISION, True)],
                         ids=["dda_flat-bf16", "dda_tree-f32", "dda_tree-bf16", "low_precision-f32",
                              "low_precision-bf16"])
@pytest.mark.parametrize("N", [2, 5, 8])
def test_allreduce_emulated(dev, orc, algo, bf16, N):
    """Every rank's buffer after lpc_allreduce_emulated equals the oracle's result of
    the same algorithm (DDA flat is bf16 only: see the next test)."""
    n = BLOCK * N * 23
    xs = [inputs.rank_buffer(inputs.LP_16MIB, r, n) for r in range(N)]
    if bf16:
        xs = [inputs.truncate_to_bf16(x) for x in xs]
    say("allreduce emulated algo=%s N=%d n=%d bf16=%s" % (lpc.ALGO_NAMES[algo], N, n, bf16))
    bufs = [to_dev(x, dev) for x in xs]
    dt = bufs[0].dtype
    ws = torch.empty(lpc.lpc_allreduce_workspace_bytes(algo, N, n, dt), dtype=torch.uint8, device=dev)
    lpc.lpc_allreduce_emulated(bufs, algo, ws)
    torch.cuda.synchronize()
    ref = _oracle_allreduce(orc, xs, algo, bf16)
    for r in range(N):
        assert_same(to_host(bufs[r]), ref, "allreduce %s rank %d" % (lpc.ALGO_NAMES[algo], r))


@pytest.mark.parametrize("N,n", [(3, 1001), (8, 8 * 977 + 5), (2, 7), (8, 4096 * 16)])
def test_allreduce_emulated_dda_flat_ragged(dev, orc, N, n):
    """DDA flat over emulated ranks at sizes that are not whole 16-byte granules (the
    copy into the ranks' buffers takes the tail element by element): every buffer
    equals the oracle's flat reduce."""
    xs = [inputs.truncate_to_bf16(inputs.normal_f32(inputs.rng(inputs.DDA_FLAT, r), n, 0.5)) for r in range(N)]
    say("allreduce emulated dda_flat ragged N=%d n=%d" % (N, n))
    bufs = [to_dev(x, dev) for x in xs]
    ws = torch.empty(lpc.lpc_allreduce_workspace_bytes(lpc.ALGO_DDA_FLAT, N, n, torch.bfloat16),
                     dtype=torch.uint8, device=dev)
    lpc.lpc_allreduce_emulated(bufs, lpc.ALGO_DDA_FLAT, ws)
    torch.cuda.synchronize()
    ref = orc.dda_flat(xs)
    for r in range(N):
        assert_same(to_host(bufs[r]), ref, "dda flat ragged rank %d" % r)


def test_allreduce_emulated_dda_flat_rejects_f32(dev):
    """DDA flat reduces bf16 only: fp32 buffers are refused before anything is
    enqueued, and the buffers are left as they were."""
    N, n = 4, BLOCK * 4 * 3
    bufs = [torch.full((n,), float(r + 1), dtype=torch.float32, device=dev) for r in range(N)]
    with pytest.raises(lpc.LpcError) as e:
        lpc.lpc_allreduce_workspace_bytes(lpc.ALGO_DDA_FLAT, N, n, torch.float32)
    assert e.value.status_name == "LPC_ERR_DTYPE"
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    with pytest.raises(lpc.LpcError) as e:
        lpc.lpc_allreduce_emulated(bufs, lpc.ALGO_DDA_FLAT, ws)
    assert e.value.status_name == "LPC_ERR_DTYPE"
    torch.cuda.synchronize()
    for r in range(N):
        assert torch.equal(bufs[r], torch.full((n,), float(r + 1), dtype=torch.float32, device=dev))


def test_allreduce_emulated_full_size_lp(dev, orc):
    """The 16 MiB workload at full size through the emulated allreduce (low precision): every
    rank's buffer equals the oracle's allreduce output."""
    N = 8
    xs = [inputs.rank_buffer(inputs.LP_16MIB, r) for r in range(N)]
    say("allreduce emulated low precision, N=8 x 16 MiB")
    bufs = [to_dev(x, dev) for x in xs]
    algo = lpc.lpc_select_algo(N, xs[0].size, torch.float32, True)
    assert algo == lpc.ALGO_LOW_PRECISION
    ws = torch.empty(lpc.lpc_allreduce_workspace_bytes(algo, N, xs[0].size, torch.float32), dtype=torch.uint8,
                     device=dev)
    lpc.lpc_allreduce_emulated(bufs, algo, ws)
    torch.cuda.synchronize()
    ref = orc.lp_allreduce(xs)["out"]
    for r in range(N):
        assert_same(to_host(bufs[r]), ref, "16 MiB LP allreduce rank %d" % r)


@pytest.mark.parametrize("N", [2, 4, 8])
def test_comm_pages_quickstart(dev, N):
    """The pages' quick-start through the torchcomms-shaped wrapper: every rank fills a
    10x20 tensor with its rank and calls allreduce(SUM) in place; every element of every
    rank must be N(N-1)/2, whichever algorithm runs (forced ones pad to their unit)."""
    import json
    import os
    from fp8_precision_allreduce_amd import comm

    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "torchcomms_quickstart_allreduce.json")))
    expect = [c["expected_every_element"] for c in gold["cases"] if c["nranks"] == N][0]
    c = comm.new_comm("lpc", dev, "main_comm", nranks=N, low_precision=True)
    runs = [(torch.float32, None), (torch.float32, lpc.ALGO_DDA_TREE), (torch.float32, lpc.ALGO_LOW_PRECISION),
            (torch.bfloat16, None), (torch.bfloat16, lpc.ALGO_DDA_FLAT), (torch.bfloat16, lpc.ALGO_LOW_PRECISION)]
    for dt, algo in runs:
        say("pages quick-start via comm N=%d dtype=%s algo=%s" % (N, dt, algo))
        ts = [torch.full((10, 20), float(r), dtype=dt, device=dev) for r in range(c.get_size())]
        used = c.allreduce(ts, comm.ReduceOp.SUM, async_op=False, algo=algo)
        if algo is not None:
            assert used == algo
        for t in ts:
            assert t.shape == (10, 20)
            assert torch.all(t.float() == expect), (dt, algo, t.float().unique())


def test_a2av_quantize_rows_70000_short_rows(dev, orc):
    """70,000 short rows (one block each): more rows than the 65,535 a grid dimension can count,
    which the flat granule kernel handles as a single 1-D range; perm from the router (with
    512-lane workgroups past 18,432 rows), checked in full against the oracle."""
    rows, row_len = 70_000, 128
    x = inputs.truncate_to_bf16(inputs.normal_f32(inputs.rng(inputs.A2AV, 2), rows * row_len, 1.0)).reshape(rows, row_len)
    dest = inputs.zipf_destinations(rows=rows)
    say("a2av quantize rows=%d row_len=%d" % (rows, row_len))
    counts = torch.empty(8, dtype=torch.int32, device=dev)
    offsets = torch.empty(8, dtype=torch.int32, device=dev)
    perm = torch.empty(rows, dtype=torch.int32, device=dev)
    lpc.lpc_a2av_route(to_dev(dest, dev), 8, counts, offsets, perm)
    codes = torch.empty((rows, row_len), dtype=torch.uint8, device=dev)
    scales = torch.empty((rows, 1), dtype=torch.float32, device=dev)
    lpc.lpc_quantize_fp8_rows(to_dev(x, dev), perm, codes, scales)
    _, _, rp = orc.a2av_route(dest, 8)
    assert_same(to_host(perm), rp, "perm")
    rc, rs = orc.quantize_rows(x, rp, bf16=True)
    assert_same(to_host(codes), rc, "rows codes")
    assert_same(to_host(scales), rs, "rows scales")


@pytest.mark.parametrize("rows,row_len", [(257, 384), (65, 2048)])
def test_a2av_quantize_rows_f32(dev, orc, rows, row_len):
    """Row gather + quantize from fp32 rows, with invalid perm entries: 3 blocks per row (each
    lane loads its own granule) and 16 blocks per row (row_len a multiple of 1,024: every
    wavefront's granules come in as one piece)."""
    x = inputs.normal_f32(inputs.rng(inputs.A2AV, 3), rows * row_len, 1.0).reshape(rows, row_len)
    _, _, perm = orc.a2av_route(inputs.zipf_destinations(rows=rows), 8)
    p = perm.copy()
    bad = (3, rows - 57)
    p[bad[0]] = -7
    p[bad[1]] = rows + 5
    say("a2av quantize rows fp32 rows=%d row_len=%d" % (rows, row_len))
    codes = torch.empty((rows, row_len), dtype=torch.uint8, device=dev)
    scales = torch.empty((rows, row_len // BLOCK), dtype=torch.float32, device=dev)
    lpc.lpc_quantize_fp8_rows(to_dev(x, dev), to_dev(p, dev), codes, scales)
    rc, rs = orc.quantize_rows(x, perm, bf16=False)
    for k in bad:
        rc[k] = 0
        rs[k] = 0.0
    assert_same(to_host(codes), rc, "fp32 rows codes")
    assert_same(to_host(scales), rs, "fp32 rows scales")
