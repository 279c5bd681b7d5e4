#!/usr/bin/env python3
"""Throughput of the linear-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one chunkwise delta-rule prefill (deltanet_prefill) of the
workload B=4, H=16, T=4096, dk=dv=128 with bf16 inputs and an fp32 state;
`value` is its throughput in tokens/s (B*T tokens per step), timed over K
back-to-back steps after W warm-up steps.  The same run times the decode
state update (deltanet_decode_step, 256 sequences x 32 heads, dk=dv=128,
512 MiB fp32 state, 10 warm-up + 1000 timed in-place steps) in GB/s, and
the CPU float64 oracle on a bounded sample of both workloads.

Inputs are seeded and synthetic (workloads.py) and resident in HBM before
timing starts.  Three copies of the prefill inputs are cycled so that
consecutive steps do not re-read the 256 MB last-level cache.  Kernel
durations come from HIP events recorded on the stream the kernels run on.

Rank count: this build runs on one GPU; --gpus above 1 exits with a message.
Prints one JSON line.
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

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
METRIC = "prefill tokens/s (delta rule, H=16,d=128,T=4K); decode state-update GB/s"
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["delta_rule_recurrent_chunkwise_amd/csrc/prefill.hip",
                  "delta_rule_recurrent_chunkwise_amd/csrc/device_common.hpp"]
DECODE_SOURCES = ["delta_rule_recurrent_chunkwise_amd/csrc/decode.hip",
                  "delta_rule_recurrent_chunkwise_amd/csrc/device_common.hpp"]


def prefill_algorithmic(B, H, T, dk, dv, in_bytes=2):
    """Bytes and flops one delta-rule prefill launch must move / do.
    Bytes: q, k, v, beta in, o out (input dtype) + the final fp32 state.
    Flops per token-head at chunk C=64: 6 dk dv (W S, Q S, K^T u) +
    2C (3 dk + 2 dv) (K K^T, Q K^T, T V-like products) + C^2/3 (the solve)."""
    C = 64
    th = B * H * T
    byts = th * in_bytes * (2 * dk + 2 * dv + 1) + B * H * dk * dv * 4
    flops = th * (6 * dk * dv + 2 * C * (3 * dk + 2 * dv) + C * C / 3)
    return byts, flops


def decode_algorithmic(N, H, dk, dv, in_bytes=2):
    """Bytes of one decode step: state read + written once (fp32), plus the
    token's q, k, v, beta in and o out."""
    heads = N * H
    return heads * (2 * dk * dv * 4 + in_bytes * (2 * dk + 2 * dv + 1))


def sources_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(name, digest):
    """HBM bytes per launch measured with rocprofv3 counters, if they were
    taken on the current kernel source; otherwise None."""
    path = os.path.join(PROFILES, name)
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sources_sha256") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


def bench_prefill(la, workloads, torch, steps, warmup, copies=3):
    w = workloads.WORKLOADS[2]
    inp = workloads.make_workload(w)
    dev = torch.device("cuda:0")
    sets = []
    for _ in range(copies):
        d = {k: v.to(dev) for k, v in inp.items()}
        d["o"] = torch.empty_like(d["v"])
        d["S"] = torch.empty(w.B, w.H, w.dk, w.dv, device=dev, dtype=torch.float32)
        sets.append(d)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    def run(d):
        la.deltanet_prefill(d["q"], d["k"], d["v"], d["beta"], S=d["S"], o=d["o"],
                            stream=stream)

    for i in range(warmup):
        run(sets[i % copies])
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        run(sets[(warmup + i) % copies])
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return w, inp, wall, kernel_ms


def bench_decode(la, workloads, torch, steps=1000, warmup=10):
    w = workloads.WORKLOADS[4]
    inp = workloads.make_workload(w)
    dev = torch.device("cuda:0")
    d = {k: v.to(dev) for k, v in inp.items()}
    S = d["S0"]
    ring = d["q"].shape[0]
    o = torch.empty(w.B, w.H, w.dv, device=dev, dtype=w.dtype)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        s = i % ring
        la.deltanet_decode_step(d["q"][s], d["k"][s], d["v"][s], d["beta"][s], S, o=o,
                                stream=stream)

    for i in range(warmup):
        step(i)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(warmup, warmup + steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    return w, inp, ev0.elapsed_time(ev1) / 1e3


def copy_probe(torch, nbytes=1 << 30, reps=5):
    """A plain device copy of known size (used to calibrate HBM counters)."""
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, device=dev, dtype=torch.float32)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return nbytes


def cpu_baseline(workloads, oracle, torch, prefill_inp, w, decode_inp, wd, budget_s=8.0):
    cores = min(len(os.sched_getaffinity(0)), 16)
    done_rows = 0
    t0 = time.perf_counter()
    for b in range(w.B):
        sub = {n: prefill_inp[n][b:b + 1].contiguous() for n in ("q", "k", "v", "beta")}
        oracle.delta_recurrent(sub["q"], sub["k"], sub["v"], sub["beta"], nthreads=cores)
        done_rows += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    tok_s = done_rows * w.T / el
    q = decode_inp
    t1 = time.perf_counter()
    oracle.delta_recurrent(q["q"][0][:, :, None], q["k"][0][:, :, None], q["v"][0][:, :, None],
                           q["beta"][0][:, :, None], None, S0=q["S0"], nthreads=cores)
    el_d = time.perf_counter() - t1
    dec_bytes = decode_algorithmic(wd.B, wd.H, wd.dk, wd.dv)
    return {
        "value": tok_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
        "sample": (f"float64 per-token recurrence over {done_rows} of {w.B} batch rows "
                   f"(H={w.H}, T={w.T}, d={w.dk}) of the prefill workload, "
                   f"{el:.1f} s wall on {cores} threads"),
        "decode": {"value": dec_bytes / el_d / 1e9, "unit": "GB/s",
                   "sample": f"one decode step over all {wd.B * wd.H} heads, {el_d:.2f} s"},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "prefill", "decode", "copy"], default="all",
                    help="run one part only (for profiler runs)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); multi-GPU sharding is not part of it.", file=sys.stderr)
        sys.exit(2)

    import torch

    import delta_rule_recurrent_chunkwise_amd as la
    import workloads

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    la.library()  # fail loudly if the HIP library is missing

    if args.only == "copy":
        n = copy_probe(torch)
        print(json.dumps({"copy_probe_bytes": n}))
        return
    if args.only == "decode":
        wd, _, el = bench_decode(la, workloads, torch, args.decode_steps)
        print(json.dumps({"decode_us_per_step": el / args.decode_steps * 1e6}))
        return

    w, pinp, wall, kms = bench_prefill(la, workloads, torch, args.steps, args.warmup)
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    ms_per_step = wall / args.steps * 1e3
    avg_kernel_s = sum(kms) / len(kms) / 1e3
    pbytes, pflops = prefill_algorithmic(B, H, T, dk, dv)
    achieved = pbytes / avg_kernel_s / 1e9
    traffic = recorded_traffic("deltanet_prefill_traffic.json", sources_digest(KERNEL_SOURCES))
    line = {
        "metric": METRIC,
        "value": B * T / (wall / args.steps),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"deltanet_prefill B={B} H={H} T={T} dk=dv={dk}, bf16 inputs, "
                               "fp32 state, 64-token chunks",
                   "B": B, "H": H, "T": T, "dk": dk, "dv": dv, "chunk": 64},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "prefill_kernel<128, BF16, PF_DELTA, 32>",
                     "algorithmic_bytes_per_launch": pbytes,
                     "avg_launch_us": avg_kernel_s * 1e6,
                     "median_launch_us": kms[len(kms) // 2] * 1e3},
        "mfma": {"achieved": pflops / avg_kernel_s / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                 "unit": "TFLOP/s", "frac": pflops / avg_kernel_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                 "algorithmic_flops_per_launch": pflops},
    }
    dinp = None
    if args.only == "all":
        wd, dinp, el = bench_decode(la, workloads, torch, args.decode_steps)
        dbytes = decode_algorithmic(wd.B, wd.H, wd.dk, wd.dv)
        gbs = dbytes * args.decode_steps / el / 1e9
        dtraffic = recorded_traffic("deltanet_decode_traffic.json", sources_digest(DECODE_SOURCES))
        line["decode"] = {
            "value": gbs, "unit": "GB/s", "steps": args.decode_steps, "warmup": 10,
            "us_per_step": el / args.decode_steps * 1e6,
            "config": {"workload": f"deltanet_decode_step N={wd.B} H={wd.H} dk=dv={wd.dk}, "
                                   "fp32 state in place, bf16 token inputs (ring of 16)"},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": dtraffic,
                         "kernel": "decode_kernel<128, 128, BF16, DEC_DELTA>",
                         "algorithmic_bytes_per_launch": dbytes},
        }
        if not args.no_cpu_baseline:
            import oracle
            line["cpu_baseline"] = cpu_baseline(workloads, oracle, torch, pinp, w, dinp, wd)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
