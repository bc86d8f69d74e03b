"""Throughput of the error-feedback top-k step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload (ResNet-50-sized flat gradient): n = 25,600,000 float32, density
0.1% (k = 25,600), gradients 99% N(0, 1e-3) + 1% Laplace(0, 0.1) at random
positions, residual carried over from earlier error-feedback steps.

A step is one tgs_topk_ef_step call: acc = residual + grad, top-k of |acc|
with the lower-index tie rule, (int32, fp32) pairs out, residual written back.
Four residual buffers and sixteen gradients (drawn on the GPU from the same
seeded mixture) rotate: consecutive steps never touch the same buffers, so no
step finds its inputs in the 256 MB Infinity Cache and every timed step streams
them from HBM, and each residual buffer meets all sixteen gradients before one
repeats.  The W warm-up steps give every residual buffer its error-feedback
history (W = 20 -> 5 steps each).

Prints one JSON line.  `roofline` covers the dominant kernel, k_step (the
whole fused step, one launch: 12n + 8k algorithmic bytes per launch), timed
with HIP events on the stream it is launched on, recorded around spans of 8
back-to-back launches: the average launch period, gaps between launches
included, without an event pair around every launch (which adds a few
microseconds of its own); `cpu_baseline` is the plain C oracle on one host core
on the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
N = 25_600_000
DENSITY = 0.001


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="before the steps, copy a 256 MiB buffer three times (a plain copy kernel of known "
                         "size, for scaling the FETCH_SIZE/WRITE_SIZE counters)")
    return ap.parse_args()


# HBM bytes per k_step launch from two rocprofv3 --pmc runs of this script
# (FETCH_SIZE, then WRITE_SIZE), each scaled by what the same counter read for
# the 256 MiB copy of --copy-calibration.  Valid only for the k_step
# source they were taken on: `source_sha256` is the hash of csrc/topk.hip then.
MEASURED_TRAFFIC = {
    "source_sha256": "5222603f03ba9a6c02403537c2e3336e2e8849018db53a84a5d5b053a0a32543",
    # FETCH_SIZE 103,058.1 KiB x (262,144 / 131,083.5: the copy's true read over its counter)
    "fetch_bytes": 211_044_472,
    # WRITE_SIZE 102,284.9 KiB x 1.0 (the copy's counter read exactly 262,144 KiB)
    "write_bytes": 104_739_737,
}


def traffic_per_launch():
    import hashlib
    if not MEASURED_TRAFFIC:
        return None
    src = os.path.join(ROOT, "top_gradient_sparsification_amd", "csrc", "topk.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if sha != MEASURED_TRAFFIC["source_sha256"]:
        return None  # the kernel changed since the counters were taken
    return MEASURED_TRAFFIC["fetch_bytes"] + MEASURED_TRAFFIC["write_bytes"]


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the per-worker step shards as independent units; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import top_gradient_sparsification_amd as tgs
    from top_gradient_sparsification_amd import workloads

    assert torch.cuda.is_available(), "no GPU visible"
    dev = torch.device("cuda:0")
    k = workloads.k_for_density(N, DENSITY)
    sets, pool = 4, 16
    print("bench: generating %d gradients of n=%d" % (pool, N), file=sys.stderr, flush=True)
    grads = [workloads.mixture_gpu(N, 1e-3, 0.01, 0.1, (workloads.CFG_RESNET50, 100, j), device=dev)
             for j in range(pool)]
    resid = [torch.zeros(N, dtype=torch.float32, device=dev) for _ in range(sets)]
    run = tgs.TopkStep(N, k, dev)
    ws = run.ws
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(t):
        run(grads[(t + t // pool) % pool], resid[t % sets])

    print("bench: warmup %d steps" % args.warmup, file=sys.stderr, flush=True)
    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    tgs.check_device_error(ws)
    fb0 = int(ws[12:16].view(torch.int32).item())  # calls whose sampled plan did not hold
    rs0 = int(ws[20:24].view(torch.int32).item())  # workgroup shares re-read (incomplete local lists)

    K = args.steps
    span = 8  # launches between two events
    nspan = max(1, K // span)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nspan + 1)]
    for e in ev:  # torch creates the HIP event on its first record
        e.record(run.stream)
    print("bench: timing %d steps" % K, file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        if i % span == 0 and i // span < nspan:
            ev[i // span].record(run.stream)
        step(args.warmup + i)
        if i + 1 == nspan * span:
            ev[nspan].record(run.stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    tgs.check_device_error(ws)
    fast = int(ws[8:12].view(torch.int32).item())  # verdict word of the last step
    fallbacks = int(ws[12:16].view(torch.int32).item()) - fb0
    rescans = int(ws[20:24].view(torch.int32).item()) - rs0
    elapsed = t1 - t0
    ms_per_step = elapsed * 1e3 / K
    main_ms = sorted(ev[j].elapsed_time(ev[j + 1]) / span for j in range(nspan))  # per launch
    main_avg_ms = sum(main_ms) / len(main_ms)
    bytes_step = 12.0 * N + 8.0 * k          # read grad + residual, write residual + k pairs
    gbps_step = bytes_step / (ms_per_step * 1e-3) / 1e9
    gbps_main = bytes_step / (main_avg_ms * 1e-3) / 1e9

    traffic = traffic_per_launch()

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        print("bench: cpu baseline (oracle, 1 core)", file=sys.stderr, flush=True)
        g = workloads.grad_resnet50(1, variant=100)
        r = workloads.grad_resnet50(2, variant=100)  # a nonzero residual of the same shape
        times = []
        for _ in range(2):
            rr = r.copy()
            c0 = time.perf_counter()
            oracle.topk_ef_step(g, rr, k)
            times.append(time.perf_counter() - c0)
        tc = min(times)
        cpu = {"value": N / tc, "unit": "elements/s", "cores": 1, "kind": "oracle",
               "sample": "2 calls of the oracle on the full n=25.6M, k=25,600 step (fastest taken), "
                         "%.2f s per call, host %s" % (tc, os.uname().machine)}

    rec = {
        "metric": "gradient elements/sec sparsified (GB/s, % HBM roofline) at n=25.6M, 0.1%",
        "value": N * K / elapsed,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "topk_ef_step n=25,600,000 k=25,600 (0.1%), grad 99% N(0,1e-3) + 1% "
                               "Laplace(0,0.1) (16 seeded GPU draws), residual from prior EF steps, "
                               "inputs resident in HBM",
                   "n": N, "k": k, "density": DENSITY},
        "gbps_step": gbps_step,
        "roofline_frac_step": gbps_step / HBM_PEAK_GBPS,
        "roofline": {"bound": "hbm", "achieved": gbps_main, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps_main / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": "k_step", "bytes_per_launch": bytes_step,
                     "avg_launch_us": main_avg_ms * 1e3, "median_launch_us": main_ms[len(main_ms) // 2] * 1e3,
                     "launches_timed": nspan * span, "timing": "HIP events around spans of %d launches" % span},
        "cpu_baseline": cpu,
        "last_step_fast_path": bool(fast == 1),
        "timed_steps_on_exact_fallback": fallbacks,
        "fallback_reasons": int(ws[16:20].view(torch.int32).item()),
        "timed_share_rescans": rescans,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
