"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with what the pages or the mathematics fix.  The
CPU test suite runs every pin on the real oracle; the mutation test runs them
on copies of the oracle with a planted mistake and expects some pin to fail.

What a pin may compare with: torch's CPU float8_e4m3fn and bfloat16 casts (an
independent library implementation of the OCP E4M3FN and bfloat16 roundings),
closed forms (exact values from power-of-two constructions), invariants,
brute force over small inputs, error bounds, and the worked example printed on
the pages (the Torchcomms quick-start: a 10x20 tensor filled with the rank,
all-reduced with SUM).
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

from fp8_precision_allreduce_amd import inputs

BLOCK = 128
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# library references (torch CPU casts)
# ---------------------------------------------------------------------------

def torch_e4m3_encode(x: np.ndarray) -> np.ndarray:
    """torch's CPU float32 -> float8_e4m3fn cast, as code bytes (non-saturating: NaN from 464 up)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def torch_e4m3_table() -> np.ndarray:
    """Value of every one of the 256 codes, decoded by torch."""
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()


def torch_bf16(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


# ---------------------------------------------------------------------------
# codec
# ---------------------------------------------------------------------------

def pin_decode_table(o):
    """All 256 codes decode to torch's values; specials from the OCP E4M3FN definition."""
    mine = o.e4m3_decode(np.arange(256, dtype=np.uint8))
    ref = torch_e4m3_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan), "NaN codes differ"
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(bits(mine[~nan]), bits(ref[~nan])), "decoded values differ from torch"
    # closed-form specials: max normal, min normal, min subnormal, one, signed zero
    assert mine[0x7E] == 448.0 and mine[0xFE] == -448.0
    assert mine[0x08] == 2.0 ** -6 and mine[0x01] == 2.0 ** -9 and mine[0x38] == 1.0
    assert bits(mine[0x80:0x81])[0] == 0x80000000
    # strictly increasing over the non-negative finite codes
    assert np.all(np.diff(mine[:0x7F].astype(np.float64)) > 0)


def _encode_probe_values() -> np.ndarray:
    table = torch_e4m3_table()[:0x7F].astype(np.float32)       # 127 non-negative finite values
    mids = ((table[:-1].astype(np.float64) + table[1:]) / 2).astype(np.float32)  # exact
    base = np.concatenate([table, mids, np.float32([464.0, 2.0 ** -10, 2.0 ** -149, 1e-40])])
    vals = [base]
    pos = base[base > 0]
    for k in range(1, 5):                                      # k ulps on either side
        vals.append((bits(base) + np.uint32(k)).view(np.float32))
        vals.append((bits(pos) - np.uint32(k)).view(np.float32))
    v = np.concatenate(vals).astype(np.float32)
    g = np.random.Generator(np.random.PCG64(7))
    rnd = g.integers(0, 2 ** 32, size=400_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    rnd = rnd[np.isfinite(rnd)]
    u = g.uniform(0, 464.0, 200_000).astype(np.float32)
    small = g.uniform(0, 2.0 ** -5, 200_000).astype(np.float32)
    v = np.concatenate([v, rnd, u, small])
    return np.concatenate([v, -v])


def pin_encode_vs_torch(o):
    """Encoder == torch's RNE cast wherever torch does not overflow (|v| < 464)."""
    v = _encode_probe_values()
    inside = np.abs(v) < 464.0
    mine = o.e4m3_encode(v[inside])
    ref = torch_e4m3_encode(v[inside])
    bad = np.nonzero(mine != ref)[0]
    assert bad.size == 0, "encode differs from torch at %r" % (v[inside][bad[:5]],)


def pin_encode_saturates(o):
    """|v| >= 448 gives +-448 (codes 0x7E / 0xFE), never NaN."""
    v = np.float32([448.0, 448.00003, 463.99997, 464.0, 500.0, 1e6, 3.4e38])
    assert np.all(o.e4m3_encode(v) == 0x7E)
    assert np.all(o.e4m3_encode(-v) == 0xFE)


def pin_encode_roundtrip(o):
    """Every finite code decodes and re-encodes to itself."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(o.e4m3_encode(o.e4m3_decode(codes)), codes)


def pin_encode_ties_even(o):
    """Every exact midpoint of two neighbouring values goes to the even code; one ulp off goes to the nearer."""
    table = torch_e4m3_table()[:0x7F].astype(np.float64)
    mids = ((table[:-1] + table[1:]) / 2).astype(np.float32)
    k = np.arange(0x7E)
    even = np.where(k % 2 == 0, k, k + 1)
    assert np.array_equal(o.e4m3_encode(mids), even.astype(np.uint8))
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    assert np.array_equal(o.e4m3_encode(up), (k + 1).astype(np.uint8))
    assert np.array_equal(o.e4m3_encode(dn), k.astype(np.uint8))
    assert np.array_equal(o.e4m3_encode(-mids), (even | 0x80).astype(np.uint8))


def pin_encode_signed_zero(o):
    """Sign is kept: -0 and tiny negatives give 0x80, +0 and tiny positives 0x00."""
    v = np.float32([0.0, -0.0, 1e-45, -1e-45, 2.0 ** -10, -(2.0 ** -10), 1e-30, -1e-30])
    assert list(o.e4m3_encode(v)) == [0x00, 0x80, 0x00, 0x80, 0x00, 0x80, 0x00, 0x80]


def pin_bf16_vs_torch(o):
    """bfloat16 round-to-nearest-even == torch's cast, on random patterns and constructed ties."""
    g = np.random.Generator(np.random.PCG64(11))
    r = g.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    r = r.view(np.float32)
    r = r[np.isfinite(r)]
    hi = g.integers(0, 2 ** 16, size=50_000, dtype=np.uint32) & np.uint32(0x7F7F)
    ties = ((hi << 16) | np.uint32(0x8000)).view(np.float32)
    near = np.concatenate([((hi << 16) | np.uint32(0x7FFF)), ((hi << 16) | np.uint32(0x8001))])
    near = near.view(np.float32)
    v = np.concatenate([r, ties, -ties, near, np.float32([0.0, -0.0, 1e-45, 3.3e38])])
    assert np.array_equal(o.bf16_rne(v), torch_bf16(v))


# ---------------------------------------------------------------------------
# blockwise quantization
# ---------------------------------------------------------------------------

def _pow2_blocks(g, nblocks: int, k_lo: int = -20, k_hi: int = 20, allow_zero_code=True):
    """Blocks of x = c * 2^k with c random finite E4M3 values and one |c| = 448 per block.

    Returns (x float32 [nblocks*128], codes, k per block)."""
    codes = g.integers(0, 0x7F, size=(nblocks, BLOCK)).astype(np.uint8)
    if not allow_zero_code:
        codes[codes == 0] = 1
    codes |= (g.integers(0, 2, size=(nblocks, BLOCK)) << 7).astype(np.uint8)
    where = g.integers(0, BLOCK, size=nblocks)
    codes[np.arange(nblocks), where] = (0x7E | (codes[np.arange(nblocks), where] & 0x80))
    table = torch_e4m3_table()
    k = g.integers(k_lo, k_hi, size=nblocks)
    x = (table[codes].astype(np.float64) * np.ldexp(1.0, k)[:, None]).astype(np.float32)
    return x.reshape(-1), codes.reshape(-1), k


def pin_quant_pow2_exact(o):
    """x = c * 2^k with max|c| = 448: the scale is exactly 2^k and the codes are exactly c."""
    g = np.random.Generator(np.random.PCG64(3))
    x, codes, k = _pow2_blocks(g, 256)
    qc, qs = o.quantize(x)
    assert np.array_equal(qs, np.ldexp(np.float32(1), k).astype(np.float32))
    assert np.array_equal(qc, codes)
    # the same values as bfloat16 (4 significant bits: exact) give the same result
    xb = bits(x) >> 16
    assert np.array_equal((xb.astype(np.uint32) << 16).view(np.float32), x)
    qc2, qs2 = o.quantize(xb.astype(np.uint16), bf16=True)
    assert np.array_equal(qc2, codes) and np.array_equal(qs2, qs)


def _brute_codes(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Brute force: nearest of all 127 torch-decoded values to fl32(x/s), ties to the even code."""
    table = torch_e4m3_table()[:0x7F].astype(np.float64)
    q = (x.reshape(-1, BLOCK) / s[:, None]).astype(np.float32).reshape(-1)  # numpy IEEE fp32 divide
    a = np.minimum(np.abs(q.astype(np.float64)), 448.0)
    d = np.abs(a[:, None] - table[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    idx = np.arange(0x7F)[None, :]
    # among equally near values take the even code
    pick = np.where(cand & (idx % 2 == 0), idx, 10_000).min(axis=1)
    pick = np.where(pick == 10_000, np.argmax(cand, axis=1), pick)
    return (pick | np.where(np.signbit(q), 0x80, 0)).astype(np.uint8)


def pin_quant_brute_force(o):
    """Small random blocks (with outliers): codes are the brute-force nearest codes of fl32(x/s)."""
    g = np.random.Generator(np.random.PCG64(5))
    x = inputs.with_outliers(g, inputs.normal_f32(g, 64 * BLOCK, 1.0), frac=0.01)
    x[:BLOCK] *= np.float32(1e-30)          # a block of tiny values
    x[BLOCK:2 * BLOCK] = np.float32(2.0 ** -140) * g.integers(-3, 4, BLOCK)  # denormal block
    qc, qs = o.quantize(x)
    amax = np.abs(x.reshape(-1, BLOCK)).max(axis=1)
    live = qs > 0
    assert np.all(live == (amax.astype(np.float64) > 448.0 * 2.0 ** -150))
    brute = _brute_codes(x.reshape(-1, BLOCK)[live].reshape(-1), qs[live])
    assert np.array_equal(qc.reshape(-1, BLOCK)[live].reshape(-1), brute)


def pin_quant_bounds(o):
    """Error of each dequantized element <= amax/28 (half the top-binade spacing 32 over 448),
    the absmax element encodes to +-448, and scale = amax/448 to within half an ulp."""
    g = np.random.Generator(np.random.PCG64(9))
    x = inputs.with_outliers(g, inputs.normal_f32(g, 512 * BLOCK, 1.0))
    qc, qs = o.quantize(x)
    deq = (torch_e4m3_table()[qc].astype(np.float64).reshape(-1, BLOCK) * qs[:, None])
    xb = x.reshape(-1, BLOCK).astype(np.float64)
    amax = np.abs(xb).max(axis=1)
    err = np.abs(deq - xb).max(axis=1)
    assert np.all(err <= amax / 28 * (1 + 2.0 ** -16))
    am = np.argmax(np.abs(xb), axis=1)
    assert np.all((qc.reshape(-1, BLOCK)[np.arange(len(am)), am] & 0x7F) == 0x7E)
    rel = np.abs(qs.astype(np.float64) - amax / 448.0) / (amax / 448.0)
    assert np.all(rel <= 2.0 ** -24 * (1 + 1e-9))


def pin_quant_zero_block(o):
    """A block of zeros (either sign) or of values whose scale underflows: scale +0, all codes 0x00."""
    x = np.zeros(3 * BLOCK, np.float32)
    x[BLOCK:2 * BLOCK] = -0.0
    x[2 * BLOCK + 5] = np.float32(1e-45)      # absmax / 448 underflows to zero
    qc, qs = o.quantize(x)
    assert np.all(qc == 0)
    assert np.array_equal(bits(qs), np.zeros(3, np.uint32))


def pin_dequant_def(o):
    """Dequantization is code value times block scale; bf16 output is torch's cast of the float output."""
    g = np.random.Generator(np.random.PCG64(13))
    codes = g.integers(0, 256, size=16 * BLOCK).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10
    scales = np.ldexp(np.float32(1), g.integers(-30, 30, 16)).astype(np.float32)
    out = o.dequantize(codes, scales)
    expect = (torch_e4m3_table()[codes].reshape(-1, BLOCK) * scales[:, None]).reshape(-1)
    assert np.array_equal(bits(out), bits(expect.astype(np.float32)))
    scales2 = inputs.normal_f32(g, 16, 1e-3)
    out2 = o.dequantize(codes, scales2)
    outb = o.dequantize(codes, scales2, bf16=True)
    assert np.array_equal(outb, torch_bf16(out2))


# ---------------------------------------------------------------------------
# low-precision allreduce
# ---------------------------------------------------------------------------

def pin_rs_pow2_exact(o):
    """Common power-of-two scales: every partial sum is exact in FP32 (<= 21 bits), so the
    rank sum equals an int64 reference; then the requantized chunk equals the quantization
    of that exact sum."""
    g = np.random.Generator(np.random.PCG64(17))
    N, nb = 8, 32
    xs, cs = [], []
    k = g.integers(-8, 8, size=nb)
    for _ in range(N):
        codes = g.integers(0, 0x7F, size=(nb, BLOCK)).astype(np.uint8)
        codes |= (g.integers(0, 2, size=(nb, BLOCK)) << 7).astype(np.uint8)
        codes[:, 0] = 0x7E
        x = (torch_e4m3_table()[codes].astype(np.float64) * np.ldexp(1.0, k)[:, None])
        xs.append(x.astype(np.float32).reshape(-1))
        cs.append(codes.reshape(-1))
    q = [o.quantize(x) for x in xs]
    for (qc, _), c in zip(q, cs):
        assert np.array_equal(qc, c)
    codes = [c for c, _ in q]
    scales = [s for _, s in q]
    # int64 reference in units of 2^(k-9): every E4M3 value is an integer multiple of 2^-9
    units = sum((torch_e4m3_table()[c].astype(np.float64) * 512).astype(np.int64) for c in cs)
    C = nb * BLOCK // N
    for r in range(N):
        s_out = o.reduce_scatter_out(codes, scales, r)
        kk = np.repeat(k, BLOCK)[r * C:(r + 1) * C]
        exact = units[r * C:(r + 1) * C].astype(np.float64) * np.ldexp(1.0, kk - 9)
        assert np.array_equal(s_out.astype(np.float64), exact)
        cc, cs_ = o.reduce_scatter_chunk(codes, scales, r)
        qc, qs = o.quantize(exact.astype(np.float32))
        assert np.array_equal(cc, qc) and np.array_equal(bits(cs_), bits(qs))


def pin_rs_rank_order(o):
    """The FP32 sum is taken in rank order 0..N-1 (brute force with numpy float32 adds),
    which differs from a pairwise-tree order on this input."""
    g = np.random.Generator(np.random.PCG64(19))
    N, n = 8, 8 * 4 * BLOCK
    xs = [inputs.normal_f32(g, n, 1.0) * np.float32(10.0 ** (p % 3)) for p in range(N)]
    q = [o.quantize(x) for x in xs]
    codes = [c for c, _ in q]
    scales = [s for _, s in q]
    table = torch_e4m3_table()
    d = [(table[c].reshape(-1, BLOCK) * s[:, None]).astype(np.float32).reshape(-1)
         for c, s in q]
    C = n // N
    tree_differs = False
    for r in range(N):
        sl = slice(r * C, (r + 1) * C)
        acc = d[0][sl].copy()
        for p in range(1, N):
            acc = (acc + d[p][sl]).astype(np.float32)
        got = o.reduce_scatter_out(codes, scales, r)
        assert np.array_equal(bits(got), bits(acc))
        # bf16 output: torch's round-to-nearest-even cast of that FP32 sum
        assert np.array_equal(o.reduce_scatter_out(codes, scales, r, bf16=True), torch_bf16(acc))
        # the requantized chunk is the blockwise quantization of that same sum
        cc, cs = o.reduce_scatter_chunk(codes, scales, r)
        qc, qs = o.quantize(acc)
        assert np.array_equal(cc, qc) and np.array_equal(bits(cs), bits(qs))
        a01, a23 = d[0][sl] + d[1][sl], d[2][sl] + d[3][sl]
        a45, a67 = d[4][sl] + d[5][sl], d[6][sl] + d[7][sl]
        tree = (a01 + a23) + (a45 + a67)
        tree_differs |= not np.array_equal(bits(tree), bits(acc))
        rev = d[N - 1][sl].copy()
        for p in range(N - 2, -1, -1):
            rev = rev + d[p][sl]
        tree_differs |= not np.array_equal(bits(rev), bits(acc))
    assert tree_differs


def pin_n1_identity(o):
    """N = 1: the reduce-scatter requantizes the dequantized buffer and gets back the same
    codes and scales bit for bit, so the output is dequant(quant(x))."""
    g = np.random.Generator(np.random.PCG64(23))
    x = inputs.with_outliers(g, inputs.normal_f32(g, 64 * BLOCK, 1.0), frac=0.01)
    res = o.lp_allreduce([x])
    assert np.array_equal(res["chunk_codes"][0], res["codes"][0])
    assert np.array_equal(bits(res["chunk_scales"][0]), bits(res["scales"][0]))
    deq = (torch_e4m3_table()[res["codes"][0]].reshape(-1, BLOCK)
           * res["scales"][0][:, None]).astype(np.float32).reshape(-1)
    assert np.array_equal(bits(res["out"]), bits(deq))


def pin_identical_buffers(o):
    """N identical buffers: for N = 2, 4 the sum is exactly N * d, codes are unchanged and the
    new scale is N * s; for N = 8 the codes are unchanged."""
    g = np.random.Generator(np.random.PCG64(29))
    x = inputs.normal_f32(g, 8 * 16 * BLOCK, 1.0)
    for N in (2, 4, 8):
        res = o.lp_allreduce([x] * N)
        codes, scales = res["codes"][0], res["scales"][0]
        C = x.size // N
        for r in range(N):
            sl = slice(r * C, (r + 1) * C)
            assert np.array_equal(res["chunk_codes"][r], codes[sl])
            if N in (2, 4):
                sb = slice(r * C // BLOCK, (r + 1) * C // BLOCK)
                assert np.array_equal(res["chunk_scales"][r], scales[sb] * np.float32(N))
        if N in (2, 4):
            deq = (torch_e4m3_table()[codes].reshape(-1, BLOCK) * scales[:, None]).reshape(-1)
            assert np.array_equal(res["out"], (deq * N).astype(np.float32))


def _ulps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in units in the last place between same-signed finite float32 arrays."""
    return np.abs(bits(a).astype(np.int64) - bits(b).astype(np.int64))


def pin_identical_buffers_n8(o):
    """N = 8 identical buffers (survey P6): every rank-order FP32 sum lies within 2 ulp of
    8 d, the requantized codes equal the original codes, and every new scale lies within
    3 ulp of 8 s.  8 d is exact (a power-of-two multiple).  The sum's bound: d + d is
    exact, and each of the six later additions errs by at most half an ulp of its result,
    which is at most half an ulp of 8 d (a quarter for the two results below 4 d): at most
    2.5 ulp of 8 d in all, so at most 2 whole ulps.  The scale's: the block absmax of the
    sums is within 2 ulp of 8 fl32(448 s), and fl32(448 s) and the division by 448 round once
    each.  Both bounds are reached: 2 and 3 ulp over 8,192 blocks with 0.1% of the values
    scaled by 100."""
    g = np.random.Generator(np.random.PCG64(31))
    N = 8
    x = inputs.normal_f32(g, N * BLOCK * 1024, 1.0)
    x[::997] *= np.float32(100.0)
    codes, scales = o.quantize(x)
    d = (torch_e4m3_table()[codes].reshape(-1, BLOCK) * scales[:, None]).reshape(-1).astype(np.float32)
    res = o.lp_allreduce([x] * N)
    C = x.size // N
    for r in range(N):
        sl, sb = slice(r * C, (r + 1) * C), slice(r * C // BLOCK, (r + 1) * C // BLOCK)
        eight_d = d[sl] * np.float32(8.0)
        assert np.array_equal(eight_d.astype(np.float64), d[sl].astype(np.float64) * 8)
        acc = o.reduce_scatter_out([codes] * N, [scales] * N, r)
        nz = eight_d != 0
        assert np.all(acc[~nz] == 0)
        assert _ulps(acc[nz], eight_d[nz]).max() <= 2, "sum of 8 identical values off by more than 2 ulp"
        assert np.array_equal(res["chunk_codes"][r], codes[sl]), "requantized codes changed"
        s8 = scales[sb] * np.float32(8.0)
        assert _ulps(res["chunk_scales"][r], s8).max() <= 3, "new scale off by more than 3 ulp"


def pin_pages_example(o):
    """The pages' quick-start: 10x20 tensors filled with the rank, all-reduced with SUM,
    give N(N-1)/2 everywhere (golden values with their citation in tests/golden)."""
    with open(os.path.join(GOLDEN, "torchcomms_quickstart_allreduce.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        N = case["nranks"]
        xs = inputs.pages_example(N)
        n = xs[0].size
        unit = BLOCK * N
        padded = -(-n // unit) * unit
        bufs = [np.concatenate([x.reshape(-1), np.zeros(padded - n, np.float32)]) for x in xs]
        out = o.lp_allreduce(bufs)["out"][:n]
        assert np.all(out == np.float32(case["expected_every_element"])), (N, np.unique(out))


def pin_e2e_bound(o):
    """Against the exact FP64 sum: |out - sum_p x_p| <= sum_p amax_p/28 + amax'/28
    + N * 2^-23 * sum_p |x_p| (two quantizations, FP32 adds), plus half a bf16 ulp for bf16."""
    g = np.random.Generator(np.random.PCG64(31))
    N, n = 8, 8 * 8 * BLOCK
    for bf16 in (False, True):
        xs = [inputs.with_outliers(g, inputs.normal_f32(g, n, 1.0), frac=0.01) for _ in range(N)]
        if bf16:
            xs = [inputs.truncate_to_bf16(x) for x in xs]
            xf = [o.bf16_to_f32(x).astype(np.float64) for x in xs]
        else:
            xf = [x.astype(np.float64) for x in xs]
        res = o.lp_allreduce(xs, bf16=bf16)
        out = o.bf16_to_f32(res["out"]) if bf16 else res["out"]
        exact = sum(xf)
        amax_sum = sum(np.repeat(np.abs(x.reshape(-1, BLOCK)).max(axis=1), BLOCK) for x in xf)
        absum = sum(np.abs(x) for x in xf)
        # absmax of each reduced block, bounded by the exact sum plus the first-stage error
        amax2 = np.repeat(np.abs(exact.reshape(-1, BLOCK)).max(axis=1), BLOCK) + \
            np.repeat(amax_sum.reshape(-1, BLOCK).max(axis=1), BLOCK) / 28 * 1.01
        bound = (amax_sum / 28 + amax2 / 28) * (1 + 2.0 ** -16) + N * 2.0 ** -23 * absum
        if bf16:
            bound = bound + np.abs(out.astype(np.float64)) * 2.0 ** -8
        assert np.all(np.abs(out.astype(np.float64) - exact) <= bound)


def pin_allgather_layout(o):
    """The all-gather output is chunk p's dequantization at [p*C, (p+1)*C); the bf16 output
    is torch's cast of the float output."""
    g = np.random.Generator(np.random.PCG64(37))
    N, C = 4, 3 * BLOCK
    cc = [g.integers(0, 0x7E, size=C).astype(np.uint8) for _ in range(N)]
    cs = [np.ldexp(np.float32(1), g.integers(-5, 5, C // BLOCK)).astype(np.float32)
          for _ in range(N)]
    out = o.allgather_dequant(cc, cs)
    table = torch_e4m3_table()
    for p in range(N):
        expect = (table[cc[p]].reshape(-1, BLOCK) * cs[p][:, None]).reshape(-1)
        assert np.array_equal(out[p * C:(p + 1) * C], expect.astype(np.float32))
    cs2 = [inputs.normal_f32(g, C // BLOCK, 1.0) for _ in range(N)]
    assert np.array_equal(o.allgather_dequant(cc, cs2, bf16=True),
                          torch_bf16(o.allgather_dequant(cc, cs2)))


def pin_compression(o):
    """Payload bytes: n codes + n/128 FP32 scales = n (1 + 4/128), i.e. 3.88:1 against fp32 and
    1.94:1 against bf16 -- within the pages' 'up to 4:1'."""
    x = inputs.normal_f32(np.random.Generator(np.random.PCG64(41)), 1024 * BLOCK, 1.0)
    c, s = o.quantize(x)
    ratio = x.nbytes / (c.nbytes + s.nbytes)
    assert abs(ratio - 4 / (1 + 4 / 128)) < 1e-12 and ratio <= 4.0


# ---------------------------------------------------------------------------
# DDA
# ---------------------------------------------------------------------------

def pin_dda_exact_ints(o):
    """bf16 inputs = small integers x 2^-k: every FP32 partial sum is exact and the final
    sum fits 8 significant bits, so the output equals an integer reference."""
    g = np.random.Generator(np.random.PCG64(43))
    N, n = 8, 4096
    ints = [g.integers(-16, 17, size=n) for _ in range(N)]
    k = 5
    bufs = [inputs.truncate_to_bf16((i * 2.0 ** -k).astype(np.float32)) for i in ints]
    out = o.dda_flat(bufs)
    expect = (sum(ints) * 2.0 ** -k).astype(np.float32)
    assert np.array_equal(o.bf16_to_f32(out), expect)


def pin_dda_rank_order(o):
    """General inputs: the FP32 rank-order sum (numpy float32 adds), cast by torch to bf16;
    and within 7 * 2^-24 relative + half a bf16 ulp of the FP64 sum."""
    bufs = inputs.dda_buffers(4)
    f = [o.bf16_to_f32(b) for b in bufs]
    acc = f[0].copy()
    for p in range(1, len(f)):
        acc = (acc + f[p]).astype(np.float32)
    out = o.dda_flat(bufs)
    assert np.array_equal(out, torch_bf16(acc))
    exact = sum(x.astype(np.float64) for x in f)
    absum = sum(np.abs(x.astype(np.float64)) for x in f)
    got = o.bf16_to_f32(out).astype(np.float64)
    assert np.all(np.abs(got - exact) <= 7 * 2.0 ** -24 * absum + np.abs(got) * 2.0 ** -8 + 1e-45)


def pin_dda_tree(o):
    """Unquantized reduce-scatter of chunk r is the owned slice of the flat reduce (bf16), and
    the numpy float32 rank-order sum (fp32)."""
    bufs = inputs.dda_buffers(1)
    N, n = len(bufs), bufs[0].size
    flat = o.dda_flat(bufs)
    C = n // N
    for r in range(N):
        assert np.array_equal(o.dda_tree_rs(bufs, r, bf16=True), flat[r * C:(r + 1) * C])
    fb = [o.bf16_to_f32(b) for b in bufs]
    for r in (0, N - 1):
        sl = slice(r * C, (r + 1) * C)
        acc = fb[0][sl].copy()
        for p in range(1, N):
            acc = acc + fb[p][sl]
        assert np.array_equal(o.dda_tree_rs(fb, r, bf16=False), acc)


# ---------------------------------------------------------------------------
# all-to-all-v
# ---------------------------------------------------------------------------

def pin_a2av_route(o):
    """Counts are the destination histogram, offsets their exclusive prefix sum, and perm a
    stable destination-major permutation (numpy's stable argsort)."""
    dest = inputs.zipf_destinations(rows=4096)
    counts, offsets, perm = o.a2av_route(dest, 8)
    assert np.array_equal(counts, np.bincount(dest, minlength=8))
    assert counts.sum() == dest.size
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)[:-1]]))
    assert np.array_equal(perm, np.argsort(dest, kind="stable"))
    assert np.array_equal(np.sort(perm), np.arange(dest.size))
    # a destination that gets no rows still has a well-defined offset
    d2 = np.array([3, 3, 0, 7, 0], np.int32)
    c2, o2, p2 = o.a2av_route(d2, 8)
    assert list(c2) == [2, 0, 0, 2, 0, 0, 0, 1] and list(o2) == [0, 2, 2, 2, 4, 4, 4, 4]
    assert list(p2) == [2, 4, 0, 1, 3]


def pin_a2av_rows(o):
    """Packed row k is the flat blockwise quantization of source row perm[k]."""
    rows, row_len = 48, 7 * BLOCK
    x = inputs.a2av_rows(rows, row_len)
    dest = inputs.zipf_destinations(rows=rows)
    _, _, perm = o.a2av_route(dest, 8)
    codes, scales = o.quantize_rows(x, perm, bf16=True)
    for k in range(rows):
        c, s = o.quantize(x[perm[k]], bf16=True)
        assert np.array_equal(codes[k], c) and np.array_equal(scales[k], s)
    # identity routing is the flat quantization of the whole matrix
    c, s = o.quantize(x.reshape(-1), bf16=True)
    ci, si = o.quantize_rows(x, np.arange(rows, dtype=np.int32), bf16=True)
    assert np.array_equal(ci.reshape(-1), c) and np.array_equal(si.reshape(-1), s)
    # fp32 rows: the same per source row
    x32 = inputs.normal_f32(np.random.Generator(np.random.PCG64(53)), rows * row_len, 1.0).reshape(rows, row_len)
    codes32, scales32 = o.quantize_rows(x32, perm, bf16=False)
    for k in range(rows):
        c, s = o.quantize(x32[perm[k]])
        assert np.array_equal(codes32[k], c) and np.array_equal(bits(scales32[k]), bits(s))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
