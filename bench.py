#!/usr/bin/env python3
"""Benchmark of the FP8 low-precision allreduce compute path on one MI355X.

Workload (the metric's configuration): N = 8 emulated ranks, 4,194,304 fp32
elements (16 MiB) per rank, N(0,1) with 0.1% outliers x100, 128-element
blocks; plus the DDA-flat reduce of 8 x 64 KiB bf16 (hidden 8192 x 4 tokens).

One step is rank 0's share of the hot path on that workload:
  1. lpc_quantize_fp8    quantize rank 0's 16 MiB buffer,
  2. lpc_rs_ag_fused     reduce rank 0's chunk over all 8 ranks' FP8 buffers,
                         requantize it, and dequantize it and the 7 peers'
                         requantized chunks into the 16 MiB fp32 output,
  3. dda_flat_reduce     8 x 64 KiB bf16 -> 64 KiB bf16.
The other ranks' quantized buffers and reduced chunks are prepared untimed,
as the peers would have produced them.  Inputs are resident in HBM when the
timed region starts.

Timing.  Every figure comes from HIP events on the stream the kernels run
on.
  * Per-kernel mean duration (value, roofline, kernels): a bounded spin
    kernel is queued first, then the launches of one kernel back to back,
    with one event before and one after them; the spin keeps the GPU behind
    the host, so the launches run back to back on the GPU and the host's
    launch cost stays out.  Mean = elapsed / launches (the pages' protocol:
    warm-up, then the mean over the measured iterations).
  * ms_per_step: one HIP graph of K steps, replayed once between two events.
The timed launches cycle through enough buffer copies (--sets) that the
256 MB Infinity Cache cannot hold them, so the kernels stream from HBM; the
256 MiB and all-to-all-v launches alternate between two copies of their
buffers.  The cache-warm DDA figure is reported beside the cold one.

value = algorithmic bytes of one fused RS+AG launch / its mean duration
(GB/s).  roofline compares it with the 8 TB/s HBM peak; traffic is the HBM
byte count per launch from rocprofv3 counters (profiles/traffic.json), null
when those counters were taken on other kernel sources.  For context the
roofline object also carries the mean duration of an empty launch timed the
same way (empty_launch_us) and the rate of the fused launch beyond it.
cpu_baseline is the CPU oracle on a bounded sample of the same share.

Extra per-kernel lines (not part of the step): the unfused reduce-scatter
and all-gather, the one-quantization low-precision reduce-scatter, the DDA
tree phases at 2 MiB bf16 per rank, the full emulated 8-rank allreduce (low
precision and DDA tree at 16 MiB, DDA flat at 64 KiB), the N=8 x 256 MiB bf16
fused launch, the fp32 fused launch at 16, 32, 64 and 128 MiB per rank, and
the all-to-all-v route, row quantize and dequantize at 16,384 x 7168 bf16.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BLOCK = 128
NRANKS = 8
MALL_BYTES = 256 * 2 ** 20


# -- algorithmic bytes (every byte read and written, scales included) -------------

def chunk_bytes(C: int) -> int:
    return C + C // BLOCK * 4                     # codes + scales of one chunk


def fused_bytes(n: int, N: int, out_size: int) -> int:
    C = n // N
    return N * chunk_bytes(C) + chunk_bytes(C) + (N - 1) * chunk_bytes(C) + n * out_size


def rs_bytes(n: int, N: int) -> int:
    C = n // N
    return N * chunk_bytes(C) + chunk_bytes(C)


def ag_bytes(n: int, N: int, out_size: int) -> int:
    return N * chunk_bytes(n // N) + n * out_size


def quantize_bytes(n: int, in_size: int) -> int:
    return n * in_size + n + n // BLOCK * 4


def dda_bytes(n: int, N: int) -> int:
    return (N + 1) * n * 2


KERNEL_SOURCES = ("lpc_device.hpp", "lpc_kernels.hip")   # every kernel's device code lives in these two


def source_digest() -> str:
    """Digest of the kernels' device sources (the counters in profiles/ are valid for
    it).  Comments and whitespace are left out, so that only a change to the code
    itself invalidates the counters."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp8_precision_allreduce_amd", "csrc")
    for f in KERNEL_SOURCES:
        with open(os.path.join(csrc, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update((f + " " + " ".join(text.split())).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec or rec.get("source_digest") != source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(xs, min_seconds: float):
    """The CPU oracle (single-threaded C) on a bounded sample of the same workload:
    rank 0's reduce-scatter chunk + all-gather dequant, repeated for ~min_seconds."""
    import oracle

    orc = oracle.default()
    N = len(xs)
    n = xs[0].size
    q = [orc.quantize(x) for x in xs]
    codes = [c for c, _ in q]
    scales = [s for _, s in q]
    chunks = [orc.reduce_scatter_chunk(codes, scales, r) for r in range(N)]
    reps = 0
    t0 = time.perf_counter()
    while True:
        orc.reduce_scatter_chunk(codes, scales, 0)
        orc.allgather_dequant([c for c, _ in chunks], [s for _, s in chunks])
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    per = el / reps
    return {
        "value": round(fused_bytes(n, N, 4) / per / 1e9, 3),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "rank 0's reduce-scatter chunk + all-gather dequant of the N=8 x 16 MiB fp32 "
                  "workload (same algorithmic bytes as one fused launch), %d repetitions in %.1f s, "
                  "single-threaded C oracle" % (reps, el),
    }


class GraphTimer:
    """Capture `count` calls of fn(i) into one HIP graph on a side stream; time replays."""

    def __init__(self, torch, fn, count: int):
        self.torch = torch
        self.count = count
        self.stream = torch.cuda.Stream()
        self.stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(self.stream):
            fn(0)                       # one eager call on the capture stream before capture
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph, stream=self.stream):
            for i in range(count):
                fn(i)
        torch.cuda.synchronize()

    def replay_us(self, reps: int = 1) -> float:
        """Mean device time per captured call over `reps` replays.  A replay runs on
        the current stream, so the events are recorded there."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            self.graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * self.count)


class BatchTimer:
    """Mean device time per launch of a batch queued behind a spin kernel."""

    def __init__(self, torch):
        self.torch = torch
        torch.cuda._sleep(1000)                  # load the spin kernel before calibrating it
        torch.cuda.synchronize()
        cycles = 20_000_000
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)                  # the events bracket GPU work only
        e0.record()
        torch.cuda._sleep(cycles)
        e1.record()
        torch.cuda.synchronize()
        self.cycles_per_us = cycles / max(e0.elapsed_time(e1) * 1e3, 1.0)

    def run(self, fn, count: int):
        """Launch fn(0..count-1) back to back; returns (mean us per launch, GPU was never idle).
        If the host's enqueueing outlasted the spin, the batch is run again with a longer spin
        (at most twice)."""
        torch = self.torch
        torch.cuda.synchronize()
        t0 = time.perf_counter()                 # host cost per launch, from a short untimed batch
        for i in range(min(count, 8)):
            fn(i)
        host_us = (time.perf_counter() - t0) * 1e6 / min(count, 8)
        torch.cuda.synchronize()
        spin_us = host_us * count * 2.0 + 1000.0
        for _ in range(3):
            es = torch.cuda.Event(enable_timing=True)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            es.record()
            torch.cuda._sleep(int(self.cycles_per_us * spin_us))
            e0.record()
            t1 = time.perf_counter()
            for i in range(count):
                fn(i)
            enqueue_us = (time.perf_counter() - t1) * 1e6
            e1.record()
            torch.cuda.synchronize()
            # the spin started no later than the host began enqueueing; it must outlast the enqueueing
            fed = es.elapsed_time(e0) * 1e3 > enqueue_us
            if fed:
                break
            spin_us = enqueue_us * 3.0 + 1000.0
        return e0.elapsed_time(e1) * 1e3 / count, fed


def stats(res, count, nbytes=None):
    us, fed = res
    d = {"us": round(us, 3), "launches": count, "gpu_fed": bool(fed)}
    if nbytes:
        d["bytes"] = nbytes
        d["gbps"] = round(nbytes / us / 1e3, 1)
    return d


class Arena:
    """The buffers of one set carved, in order, from a single allocation (4 KiB
    aligned), as the library's own emulated-allreduce workspace is laid out.
    The N emulated ranks' buffers share one GPU's HBM, which a real rank's
    peers (each in its own GPU's memory) do not.  Allocated one tensor at a
    time, the fused kernel's time at 16 MiB depended on where the allocator
    placed them: 4.88 to 5.59 us per launch across placements and boxes, and
    up to 10% apart between two placements on one box.  Packed into one
    allocation it measured 4.85 to 5.01 us on the same boxes."""

    ALIGN = 4096

    def __init__(self, torch, dev, sizes):
        self.torch = torch
        total = sum(-(-b // self.ALIGN) * self.ALIGN for b in sizes)
        self.buf = torch.empty(total, dtype=torch.uint8, device=dev)
        self.off = 0

    def take(self, numel, dtype):
        nbytes = numel * self.torch.empty((), dtype=dtype).element_size()
        t = self.buf[self.off:self.off + nbytes].view(dtype)
        self.off += -(-nbytes // self.ALIGN) * self.ALIGN
        return t


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=16, help="buffer copies of the 16 MiB workload cycled through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the per-kernel lines outside the step (256 MiB bf16, fused by size, all-to-all-v)")
    ap.add_argument("--dda-sets", type=int, default=0,
                    help="DDA buffer sets cycled through (0: enough to exceed the 256 MB cache)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 64 MiB device copy (calibration for counter runs)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py: this benchmark runs on one GPU only (the N ranks are emulated as N buffers "
              "in one GPU's HBM); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    from fp8_precision_allreduce_amd import inputs, lpc

    def log(msg):
        print("[bench] " + msg, file=sys.stderr, flush=True)

    lpc.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    N = NRANKS
    n = inputs.WORKLOADS[inputs.LP_16MIB]["n"]
    C = n // N
    log("generating workload: N=%d x %d fp32 per rank" % (N, n))
    xs_host = [inputs.rank_buffer(inputs.LP_16MIB, r) for r in range(N)]

    # -- untimed setup: every rank's quantized buffer and reduced chunk ------------------
    xs = [torch.from_numpy(x).to(dev) for x in xs_host]
    codes = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(N)]
    scales = [torch.empty(n // BLOCK, dtype=torch.float32, device=dev) for _ in range(N)]
    for r in range(N):
        lpc.lpc_quantize_fp8(xs[r], codes[r], scales[r])
    cc = [torch.empty(C, dtype=torch.uint8, device=dev) for _ in range(N)]
    cs = [torch.empty(C // BLOCK, dtype=torch.float32, device=dev) for _ in range(N)]
    for r in range(N):
        lpc.lpc_reduce_scatter_chunk(codes, scales, r, cc[r], cs[r])
    out_ref = torch.empty(n, dtype=torch.float32, device=dev)
    lpc.lpc_allgather_dequant(cc, cs, out_ref)
    torch.cuda.synchronize()

    S = max(1, args.sets)
    sets = []
    u8, f32 = torch.uint8, torch.float32
    for _ in range(S):
        a = Arena(torch, dev, [n * 4] + [n, n // BLOCK * 4] * N + [C, C // BLOCK * 4] * (2 * N + 1) + [n * 4])
        b = dict(x=a.take(n, f32))
        b["codes"], b["scales"] = [], []
        for r in range(N):
            b["codes"].append(a.take(n, u8))
            b["scales"].append(a.take(n // BLOCK, f32))
        b["peer_c"], b["peer_s"], b["all_c"], b["all_s"] = [None], [None], [], []
        for r in range(N):
            if r > 0:
                b["peer_c"].append(a.take(C, u8))
                b["peer_s"].append(a.take(C // BLOCK, f32))
            b["all_c"].append(a.take(C, u8))
            b["all_s"].append(a.take(C // BLOCK, f32))
        b["own_c"], b["own_s"], b["out"] = a.take(C, u8), a.take(C // BLOCK, f32), a.take(n, f32)
        b["x"].copy_(xs[0])
        for r in range(N):
            b["codes"][r].copy_(codes[r])
            b["scales"][r].copy_(scales[r])
            b["all_c"][r].copy_(cc[r])
            b["all_s"][r].copy_(cs[r])
            if r > 0:
                b["peer_c"][r].copy_(cc[r])
                b["peer_s"][r].copy_(cs[r])
        sets.append(b)
    set_bytes = sum(t.numel() * t.element_size() for b in sets[:1] for k, v in b.items()
                    for t in (v if isinstance(v, list) else [v]) if t is not None)

    # DDA flat sets: 8 ranks x (hidden 8192 x T) bf16 + output, enough to exceed the cache
    dda_host = {T: inputs.dda_buffers(T) for T in inputs.DDA_TOKENS}

    def dda_sets(T, count):
        m = dda_host[T][0].size
        pool = torch.empty((count, N + 1, m), dtype=torch.bfloat16, device=dev)
        src = torch.stack([torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16) for b in dda_host[T]])
        pool[:, :N].copy_(src.unsqueeze(0).expand(count, N, m))
        return pool

    def dda_cold_count(T):
        if args.dda_sets > 0:
            return args.dda_sets
        m = dda_host[T][0].size
        return max(64, -(-2 * MALL_BYTES // dda_bytes(m, N)))

    pools = {T: dda_sets(T, dda_cold_count(T)) for T in inputs.DDA_TOKENS}
    torch.cuda.synchronize()

    # -- the kernels --------------------------------------------------------------------------
    def quantize(i):
        b = sets[i % S]
        lpc.lpc_quantize_fp8(b["x"], b["codes"][0], b["scales"][0])

    def fused(i):
        b = sets[i % S]
        lpc.lpc_rs_ag_fused(b["codes"], b["scales"], 0, b["own_c"], b["own_s"], b["peer_c"], b["peer_s"],
                            b["out"])

    def rs_chunk(i):
        b = sets[i % S]
        lpc.lpc_reduce_scatter_chunk(b["codes"], b["scales"], 0, b["own_c"], b["own_s"])

    def allgather(i):
        b = sets[i % S]
        lpc.lpc_allgather_dequant(b["all_c"], b["all_s"], b["out"])

    def dda(T, i):
        pool = pools[T]
        k = i % pool.shape[0]
        lpc.dda_flat_reduce([pool[k, p] for p in range(N)], pool[k, N])

    def step(i):
        quantize(i)
        fused(i)
        dda(4, i)

    # -- warmup (eager), then graph capture of the K steps -------------------------------------------
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    log("capturing graphs (%d steps)" % K)
    g_step = GraphTimer(torch, step, K)
    g_step.replay_us(1)                     # warm replay, untimed

    # -- timed region: exactly K steps ------------------------------------------------------------------
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    step_us = g_step.replay_us(1)
    wall_s = time.perf_counter() - t_wall
    total_ms = step_us * K / 1e3

    # -- per-kernel mean durations, each batch after a cache-evicting replay ------------------------------
    timer = BatchTimer(torch)
    L = max(K, 2 * S)

    def timed(fn, count, nbytes=None):
        g_step.replay_us(1)                 # >1 GB of other traffic: the batch starts cache-cold
        return stats(timer.run(fn, count), count, nbytes)

    fb = fused_bytes(n, N, 4)
    kernels = {
        "rs_ag_fused_f32_16MiB": timed(fused, L, fb),
        "quantize_f32_16MiB": timed(quantize, L, quantize_bytes(n, 4)),
        "reduce_scatter_chunk_16MiB": timed(rs_chunk, L, rs_bytes(n, N)),
        "allgather_dequant_f32_16MiB": timed(allgather, L, ag_bytes(n, N, 4)),
    }
    dda_res = {}
    for T in inputs.DDA_TOKENS:
        m = dda_host[T][0].size
        cnt = min(K, pools[T].shape[0])
        r = timed(lambda i, T=T: dda(T, i), cnt, dda_bytes(m, N))
        r["buffer_sets"] = cnt
        dda_res["%dKiB" % (m * 2 // 1024)] = r
    warm = stats(timer.run(lambda i: dda(4, i % 4), K), K)
    dda_res["64KiB"]["us_warm"] = warm["us"]
    # the same batch of launches of a kernel that does nothing (one lane, no memory): the fixed cost
    # every launch above pays before it moves a byte
    floor_us = timer.run(lambda i: torch.cuda._sleep(0), L)[0]

    # -- the same two headline kernels as graph replays (back to back inside one graph) --------------------
    g_fused = GraphTimer(torch, fused, L)
    g_dda = GraphTimer(torch, lambda i: dda(4, i), pools[4].shape[0])
    g_fused.replay_us(1)
    g_dda.replay_us(1)
    kernels["rs_ag_fused_f32_16MiB"]["graph_replay_us"] = round(g_fused.replay_us(3), 3)
    dda_res["64KiB"]["graph_replay_us"] = round(g_dda.replay_us(3), 3)

    # -- every launch and replay left the eager result in place --------------------------------------------
    for b in sets:
        assert torch.equal(b["own_c"], cc[0]), "reduced chunk differs from the eager result"
        assert torch.equal(b["own_s"].view(torch.int32), cs[0].view(torch.int32)), "chunk scales differ"
        assert torch.equal(b["out"].view(torch.int32), out_ref.view(torch.int32)), "output differs"
        assert torch.equal(b["codes"][0], codes[0]), "quantized buffer differs"
    for T in inputs.DDA_TOKENS:
        pool = pools[T]
        ref = torch.empty_like(pool[0, N])
        lpc.dda_flat_reduce([pool[0, p] for p in range(N)], ref)
        written = pool[:min(K, pool.shape[0]), N]
        assert torch.equal(written.view(torch.int16), ref.view(torch.int16).expand_as(written)), \
            "DDA flat output differs"
    torch.cuda.synchronize()

    # -- next rows: one-quantization reduce-scatter, DDA tree, the emulated 8-rank allreduce ---------------
    def lp_rs(i):
        b = sets[i % S]
        lpc.lpc_reduce_scatter(b["codes"], b["scales"], 0, b["rs_out"])

    for b in sets:
        b["rs_out"] = torch.empty(C, dtype=torch.float32, device=dev)
    kernels["lp_reduce_scatter_f32_16MiB"] = timed(lp_rs, L, N * chunk_bytes(C) + C * 4)
    nt = 8 * 2 ** 20 // 16 * 2                            # 2 MiB of bf16 per rank
    tree_sets = [[torch.randn(nt, device=dev).to(torch.bfloat16) for _ in range(N)] for _ in range(S)]
    tree_chunks = [[torch.empty(nt // N, dtype=torch.bfloat16, device=dev) for _ in range(N)] for _ in range(S)]
    tree_out = [torch.empty(nt, dtype=torch.bfloat16, device=dev) for _ in range(S)]
    kernels["dda_tree_rs_bf16_2MiB"] = timed(
        lambda i: lpc.dda_tree_reduce_scatter(tree_sets[i % S], 0, tree_chunks[i % S][0]), L,
        N * (nt // N) * 2 + (nt // N) * 2)
    kernels["dda_tree_ag_bf16_2MiB"] = timed(
        lambda i: lpc.dda_tree_allgather(tree_chunks[i % S], tree_out[i % S]), L, nt * 2 * 2)
    for algo, name, dt in ((lpc.ALGO_LOW_PRECISION, "low_precision", torch.float32),
                           (lpc.ALGO_DDA_TREE, "dda_tree", torch.float32)):
        ar_bufs = [[b["out"]] + [torch.empty(n, dtype=dt, device=dev) for _ in range(N - 1)] for b in sets[:4]]
        for bl in ar_bufs:
            for t in bl:
                t.copy_(xs[0])
        ws = torch.empty(lpc.lpc_allreduce_workspace_bytes(algo, N, n, dt), dtype=torch.uint8, device=dev)
        r = stats(timer.run(lambda i: lpc.lpc_allreduce_emulated(ar_bufs[i % len(ar_bufs)], algo, ws), 8), 8)
        r["what"] = "all 8 ranks' shares in place, one launch per step"
        kernels["allreduce_emulated_%s_n8_16MiB" % name] = r
        del ar_bufs, ws
    del tree_sets, tree_chunks, tree_out
    # the small-message allreduce: DDA flat over the 8 emulated ranks at 64 KiB bf16 per rank
    m64 = inputs.HIDDEN * 4
    flat_sets = [[torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16) for b in dda_host[4]]
                 for _ in range(16)]
    ws_flat = torch.empty(lpc.lpc_allreduce_workspace_bytes(lpc.ALGO_DDA_FLAT, N, m64, torch.bfloat16),
                          dtype=torch.uint8, device=dev)
    r = stats(timer.run(lambda i: lpc.lpc_allreduce_emulated(flat_sets[i % len(flat_sets)], lpc.ALGO_DDA_FLAT,
                                                             ws_flat), 32), 32)
    r["what"] = "all 8 ranks' shares in place: one reduce launch and one copy launch"
    kernels["allreduce_emulated_dda_flat_n8_64KiB"] = r
    del flat_sets, ws_flat

    f_us = kernels["rs_ag_fused_f32_16MiB"]["us"]
    value = fb / (f_us * 1e-6) / 1e9
    del g_step, g_fused, g_dda, pools
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    # -- extra per-kernel lines: 256 MiB bf16 per rank, all-to-all-v rows ------------------------------
    if not args.no_extra:
        log("256 MiB bf16 per rank (device-generated) and all-to-all-v rows")
        # Two copies of each large workload, used in turn: one copy (about 1.4 GiB for the 256 MiB
        # fused launch) already exceeds the 256 MB Infinity Cache, but a kernel relaunched on the
        # same buffers still finds part of them there (quantize bf16: 58 against 70 us).
        COPIES = 2
        n4 = inputs.WORKLOADS[inputs.LP_256MIB_BF16]["n"]
        C4 = n4 // N
        sets4 = []
        for k in range(COPIES):
            a4 = Arena(torch, dev, [n4 * 2] + [n4, n4 // BLOCK * 4] * N + [C4, C4 // BLOCK * 4] * (N + 1) + [n4 * 2])
            b4 = dict(x=a4.take(n4, torch.bfloat16), codes=[], scales=[], cc=[], cs=[])
            for r in range(N):
                b4["codes"].append(a4.take(n4, torch.uint8))
                b4["scales"].append(a4.take(n4 // BLOCK, torch.float32))
            for r in range(N):
                b4["cc"].append(a4.take(C4, torch.uint8))
                b4["cs"].append(a4.take(C4 // BLOCK, torch.float32))
            b4["oc"], b4["os"] = a4.take(C4, torch.uint8), a4.take(C4 // BLOCK, torch.float32)
            b4["out"] = a4.take(n4, torch.bfloat16)
            if k == 0:
                for r in range(N):
                    x4 = inputs.device_rank_buffer(inputs.LP_256MIB_BF16, r, dev)
                    lpc.lpc_quantize_fp8(x4, b4["codes"][r], b4["scales"][r])
                    if r == 0:
                        b4["x"].copy_(x4)
                    del x4
                for r in range(N):
                    lpc.lpc_reduce_scatter_chunk(b4["codes"], b4["scales"], r, b4["cc"][r], b4["cs"][r])
            else:
                for key in ("x",):
                    b4[key].copy_(sets4[0][key])
                for key in ("codes", "scales", "cc", "cs"):
                    for dst, src in zip(b4[key], sets4[0][key]):
                        dst.copy_(src)
            sets4.append(b4)
        torch.cuda.synchronize()

        def fused4(i):
            b = sets4[i % COPIES]
            lpc.lpc_rs_ag_fused(b["codes"], b["scales"], 0, b["oc"], b["os"], [None] + b["cc"][1:],
                                [None] + b["cs"][1:], b["out"])

        def quantize4(i):
            b = sets4[i % COPIES]
            lpc.lpc_quantize_fp8(b["x"], b["codes"][0], b["scales"][0])

        for i in range(2 * COPIES):
            fused4(i)
            quantize4(i)
        torch.cuda.synchronize()
        kernels["rs_ag_fused_bf16_256MiB"] = stats(timer.run(fused4, 20), 20, fused_bytes(n4, N, 2))
        kernels["quantize_bf16_256MiB"] = stats(timer.run(quantize4, 20), 20, quantize_bytes(n4, 2))
        for b in sets4:
            assert torch.equal(b["oc"], sets4[0]["cc"][0]), "256 MiB bf16: reduced chunk differs"
        del sets4, b4, a4
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

        # The fused kernel against message size: fp32, N=8, values as in the 16 MiB workload.  The
        # launch's fixed cost weighs less as the message grows.  Copies are cycled so that together
        # they hold at least three times the Infinity Cache.
        sizes = {}
        for mib in (16, 32, 64, 128):
            ns = mib * 2 ** 20 // 4
            Cs = ns // N
            layout = [ns, ns // BLOCK * 4] * N + [Cs, Cs // BLOCK * 4] * (N + 1) + [ns * 4]
            copies = max(2, -(-3 * MALL_BYTES // sum(layout)))
            sets_s = []
            for k in range(copies):
                a_s = Arena(torch, dev, layout)
                b_s = dict(codes=[], scales=[], cc=[], cs=[])
                for r in range(N):
                    b_s["codes"].append(a_s.take(ns, torch.uint8))
                    b_s["scales"].append(a_s.take(ns // BLOCK, torch.float32))
                for r in range(N):
                    b_s["cc"].append(a_s.take(Cs, torch.uint8))
                    b_s["cs"].append(a_s.take(Cs // BLOCK, torch.float32))
                b_s["oc"], b_s["os"] = a_s.take(Cs, torch.uint8), a_s.take(Cs // BLOCK, torch.float32)
                b_s["out"] = a_s.take(ns, torch.float32)
                if k == 0:
                    for r in range(N):
                        xs_r = inputs.device_rank_buffer(inputs.LP_16MIB, r, dev, n=ns)
                        lpc.lpc_quantize_fp8(xs_r, b_s["codes"][r], b_s["scales"][r])
                        del xs_r
                    for r in range(N):
                        lpc.lpc_reduce_scatter_chunk(b_s["codes"], b_s["scales"], r, b_s["cc"][r], b_s["cs"][r])
                else:
                    for key in ("codes", "scales", "cc", "cs"):
                        for dst, src in zip(b_s[key], sets_s[0][key]):
                            dst.copy_(src)
                sets_s.append(b_s)
            torch.cuda.synchronize()

            def fused_s(i, sets_s=sets_s):
                b = sets_s[i % len(sets_s)]
                lpc.lpc_rs_ag_fused(b["codes"], b["scales"], 0, b["oc"], b["os"], [None] + b["cc"][1:],
                                    [None] + b["cs"][1:], b["out"])

            for i in range(2 * copies):
                fused_s(i)
            torch.cuda.synchronize()
            d = stats(timer.run(fused_s, 40), 40, fused_bytes(ns, N, 4))
            d["frac"] = round(d["gbps"] / HBM_PEAK_GBPS, 4)
            d["copies"] = copies
            sizes["%dMiB" % mib] = d
            for b in sets_s:
                assert torch.equal(b["oc"], sets_s[0]["cc"][0]), "fused %d MiB: reduced chunk differs" % mib
            del sets_s, b_s, a_s, fused_s
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        kernels["rs_ag_fused_f32_by_size"] = sizes

        rows, row_len = inputs.A2AV_ROWS, inputs.A2AV_ROW_LEN
        m5 = rows * row_len
        xr0 = torch.from_numpy(inputs.a2av_rows().view(np.int16)).to(dev).view(torch.bfloat16)
        dest = torch.from_numpy(inputs.zipf_destinations()).to(dev)
        counts = torch.empty(N, dtype=torch.int32, device=dev)
        offsets = torch.empty(N, dtype=torch.int32, device=dev)
        perm = torch.empty(rows, dtype=torch.int32, device=dev)
        lpc.lpc_a2av_route(dest, N, counts, offsets, perm)
        sets5 = []
        for k in range(COPIES):
            a5 = Arena(torch, dev, [m5 * 2, m5, m5 // BLOCK * 4, m5 * 2])
            b5 = dict(x=a5.take(m5, torch.bfloat16).view(rows, row_len),
                      codes=a5.take(m5, torch.uint8).view(rows, row_len),
                      scales=a5.take(m5 // BLOCK, torch.float32).view(rows, row_len // BLOCK),
                      back=a5.take(m5, torch.bfloat16).view(rows, row_len))
            b5["x"].copy_(xr0)
            lpc.lpc_quantize_fp8_rows(b5["x"], perm, b5["codes"], b5["scales"])
            lpc.lpc_dequantize_fp8(b5["codes"], b5["scales"], b5["back"])
            sets5.append(b5)
        del xr0
        torch.cuda.synchronize()
        kernels["a2av_route_16384"] = stats(timer.run(
            lambda i: lpc.lpc_a2av_route(dest, N, counts, offsets, perm), 20), 20, rows * 4 * 2 + N * 8)
        kernels["a2av_quantize_rows_bf16"] = stats(timer.run(
            lambda i: lpc.lpc_quantize_fp8_rows(sets5[i % COPIES]["x"], perm, sets5[i % COPIES]["codes"],
                                                sets5[i % COPIES]["scales"]), 20), 20,
            quantize_bytes(m5, 2) + rows * 4)
        kernels["a2av_dequantize_bf16"] = stats(timer.run(
            lambda i: lpc.lpc_dequantize_fp8(sets5[i % COPIES]["codes"], sets5[i % COPIES]["scales"],
                                             sets5[i % COPIES]["back"]), 20), 20, m5 + m5 // BLOCK * 4 + m5 * 2)
        del sets5, b5, a5
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    if args.copy_probe:
        # a plain copy of known size (64 MiB read, 64 MiB written): the DDA-tree gather copy
        src = [torch.ones(2 * 2 ** 20, dtype=torch.float32, device=dev) for _ in range(N)]
        dst = torch.empty(16 * 2 ** 20, dtype=torch.float32, device=dev)
        for _ in range(5):
            lpc.dda_tree_allgather(src, dst)
        torch.cuda.synchronize()

    traffic = traffic_from_profiles("rs_ag_fused_kernel<8,float>")
    result = {
        "metric": "FP8 RS+AG reduce GB/s & % of HBM peak (16MB/rank, N=8); DDA-flat µs @64KB",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / K, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) fp32 with 0.1% outliers x100; DDA: seeded N(0,0.5) bf16); FP8 E4M3 storage, FP32 arithmetic",
        "config": {
            "workload": "lp_allreduce_n8_16MiB_f32 + dda_flat_n8_64KiB_bf16: rank 0's share of an N=8 FP8 "
                        "low-precision allreduce, 4,194,304 fp32 per rank, 128-element blocks, E4M3 + FP32 "
                        "scales; DDA-flat reduce of 8 x 32,768 bf16",
            "nranks": N, "elems_per_rank": n, "block": BLOCK,
            "step": "quantize + fused RS+AG + DDA flat 64 KiB",
            "buffer_sets": S, "set_bytes": set_bytes, "hbm_resident": True,
            "timing": "kernels: back-to-back batch behind a spin kernel, HIP events around it; step: HIP graph replay",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(value, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(value / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": "rs_ag_fused_kernel<8,float>",
            "bytes_per_launch": fb,
            "mean_us": round(f_us, 3),
            "launches": kernels["rs_ag_fused_f32_16MiB"]["launches"],
            # context: an empty launch's share of mean_us on this GPU, and the rate of the rest
            "empty_launch_us": round(floor_us, 3),
            "beyond_empty_launch_gbps": round(fb / max(f_us - floor_us, 1e-3) / 1e3, 1),
        },
        "kernels": kernels,
        "dda_flat_n8_bf16": dda_res,
        "dda_flat_us_64KiB": dda_res["64KiB"]["us"],
        "step_wall_s": round(wall_s, 6),
        "source_digest": source_digest(),
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(xs_host, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
