#!/usr/bin/env python3
"""Benchmark of the FP8 low-precision allreduce compute path on one MI355X.

Workload (the metric's configuration): N = 8 emulated ranks, 4,194,304 fp32
elements (16 MiB) per rank, N(0,1) with 0.1% outliers x100, 128-element
blocks.  One step is rank 0's share of the low-precision allreduce: quantize
its buffer (lpc_quantize_fp8), then the fused reduce-scatter + all-gather
(lpc_rs_ag_fused: reduce the owned chunk over all 8 ranks' FP8 buffers,
requantize it, dequantize it and the 7 peers' requantized chunks into the
output).  The other ranks' quantized buffers and reduced chunks are prepared
untimed, as the peers would have produced them.

Inputs are resident in HBM when timing starts.  The step cycles through
enough copies of every buffer (--sets) that the 256 MB Infinity Cache cannot
hold them, so kernels stream from HBM; --sets 1 gives the cache-warm figure.

value = algorithmic bytes of one fused RS+AG launch / its mean duration
(GB/s), durations from HIP events recorded around each launch on the stream
the kernels run on.  The roofline object compares it with the 8 TB/s HBM
peak.  DDA-flat latency (8 x 64 KiB bf16) is reported alongside.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BLOCK = 128


def fused_bytes(n: int, N: int, out_size: int) -> int:
    C = n // N
    chunk = C + C // BLOCK * 4                   # codes + scales of one chunk
    return N * chunk + chunk + (N - 1) * chunk + n * out_size


def quantize_bytes(n: int, in_size: int) -> int:
    return n * in_size + n + n // BLOCK * 4


def dda_bytes(n: int, N: int) -> int:
    return (N + 1) * n * 2


def source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp8_precision_allreduce_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=16, help="buffer copies cycled through (1 = cache-warm)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--dda-steps", type=int, default=200)
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (the N ranks are emulated as N buffers "
              "in one GPU's HBM); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from fp8_precision_allreduce_amd import inputs, lpc

    lpc.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    N = 8
    n = inputs.CONFIGS[3]["n"]
    C = n // N
    print("[bench] generating workload: N=%d x %d fp32 per rank" % (N, n), file=sys.stderr, flush=True)
    xs_host = [inputs.rank_buffer(3, r) for r in range(N)]

    # -- untimed setup: every rank's quantized buffer and reduced chunk -------------
    xs = [torch.from_numpy(x).to(dev) for x in xs_host]
    codes = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(N)]
    scales = [torch.empty(n // BLOCK, dtype=torch.float32, device=dev) for _ in range(N)]
    for r in range(N):
        lpc.lpc_quantize_fp8(xs[r], codes[r], scales[r])
    cc = [torch.empty(C, dtype=torch.uint8, device=dev) for _ in range(N)]
    cs = [torch.empty(C // BLOCK, dtype=torch.float32, device=dev) for _ in range(N)]
    for r in range(N):
        lpc.lpc_reduce_scatter_chunk(codes, scales, r, cc[r], cs[r])
    torch.cuda.synchronize()

    # -- buffer sets cycled through by the timed steps -----------------------------------
    S = max(1, args.sets)
    sets = []
    for _ in range(S):
        sets.append(dict(
            x=xs[0].clone(),
            codes=[c.clone() for c in codes],
            scales=[s.clone() for s in scales],
            peer_c=[None] + [c.clone() for c in cc[1:]],
            peer_s=[None] + [s.clone() for s in cs[1:]],
            own_c=torch.empty(C, dtype=torch.uint8, device=dev),
            own_s=torch.empty(C // BLOCK, dtype=torch.float32, device=dev),
            out=torch.empty(n, dtype=torch.float32, device=dev),
        ))
    torch.cuda.synchronize()

    def step(i, ev=None):
        b = sets[i % S]
        if ev is not None:
            ev[0].record(stream)
        lpc.lpc_quantize_fp8(b["x"], b["codes"][0], b["scales"][0], stream=stream)
        if ev is not None:
            ev[1].record(stream)
        lpc.lpc_rs_ag_fused(b["codes"], b["scales"], 0, b["own_c"], b["own_s"], b["peer_c"], b["peer_s"],
                            b["out"], stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # -- timed region: K steps, events around each launch ------------------------------------
    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(K):
        step(args.warmup + i, evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    q_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    f_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])

    # correctness spot check of the last step against the untimed reference chunk
    last = sets[(args.warmup + K - 1) % S]
    assert torch.equal(last["own_c"], cc[0]), "fused kernel's reduced chunk changed between runs"

    fb = fused_bytes(n, N, 4)
    qb = quantize_bytes(n, 4)
    f_mean_s = float(f_ms.mean()) * 1e-3
    q_mean_s = float(q_ms.mean()) * 1e-3
    value = fb / f_mean_s / 1e9

    # -- back-to-back launches (no events between): loop-average duration ---------------------
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(K):
        b = sets[i % S]
        lpc.lpc_rs_ag_fused(b["codes"], b["scales"], 0, b["own_c"], b["own_s"], b["peer_c"], b["peer_s"],
                            b["out"], stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    f_loop_us = e0.elapsed_time(e1) / K * 1e3

    # -- DDA flat, 8 ranks x 64 KiB bf16 (hidden 8192 x 4 tokens) ------------------------------
    dda = {}
    for T in inputs.DDA_TOKENS:
        bufs_h = inputs.dda_buffers(T)
        m = bufs_h[0].size
        DS = max(1, min(S * 8, 64))
        dsets = [([torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16) for b in bufs_h],
                  torch.empty(m, dtype=torch.bfloat16, device=dev)) for _ in range(DS)]
        for i in range(20):
            lpc.dda_flat_reduce(dsets[i % DS][0], dsets[i % DS][1], stream=stream)
        torch.cuda.synchronize()
        D = args.dda_steps
        dev_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(D)]
        for i in range(D):
            bset, o = dsets[i % DS]
            dev_ev[i][0].record(stream)
            lpc.dda_flat_reduce(bset, o, stream=stream)
            dev_ev[i][1].record(stream)
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) for a, b in dev_ev]) * 1e3
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for i in range(D):
            bset, o = dsets[i % DS]
            lpc.dda_flat_reduce(bset, o, stream=stream)
        a1.record(stream)
        torch.cuda.synchronize()
        dda["%dKiB" % (m * 2 // 1024)] = {
            "event_us_mean": round(float(us.mean()), 3),
            "event_us_median": round(float(np.median(us)), 3),
            "loop_us_per_call": round(a0.elapsed_time(a1) / D * 1e3, 3),
            "bytes": dda_bytes(m, 8),
        }
        del dsets

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
        "dtype": "fp8-e4m3/f32",
        "data": "synthetic (seeded N(0,1) fp32 with 0.1% outliers x100)",
        "config": {
            "workload": "lp_allreduce_n8_16MiB_f32: one rank's share of an N=8 FP8 low-precision "
                        "allreduce, 4,194,304 fp32 per rank, 128-element blocks, E4M3 + FP32 scales",
            "nranks": N, "elems_per_rank": n, "block": BLOCK, "step": "quantize + fused RS+AG",
            "buffer_sets": S, "hbm_resident": True,
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
            "mean_us": round(f_mean_s * 1e6, 3),
        },
        "kernels": {
            "rs_ag_fused": {"event_us_mean": round(float(f_ms.mean()) * 1e3, 3),
                            "event_us_median": round(float(np.median(f_ms)) * 1e3, 3),
                            "event_us_min": round(float(f_ms.min()) * 1e3, 3),
                            "loop_us_per_launch": round(f_loop_us, 3),
                            "bytes": fb, "gbps": round(value, 2)},
            "quantize_f32": {"event_us_mean": round(q_mean_s * 1e6, 3),
                             "event_us_median": round(float(np.median(q_ms)) * 1e3, 3),
                             "bytes": qb, "gbps": round(qb / q_mean_s / 1e9, 2)},
        },
        "dda_flat_n8_bf16": dda,
        "dda_flat_us_64KiB": dda.get("64KiB", {}).get("event_us_mean"),
        "source_digest": source_digest(),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(xs_host, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
