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
_CSRC = "delta_rule_recurrent_chunkwise_amd/csrc/"
PREFILL_SOURCES = [_CSRC + "prefill_pipe.hip", _CSRC + "device_common.hpp", _CSRC + "launch.hpp"]
DECODE_SOURCES = [_CSRC + "decode.hip", _CSRC + "device_common.hpp", _CSRC + "launch.hpp"]
# Symbol substrings of the two timed kernels (as rocprofv3 lists them) and the
# profile summaries that record their counters.
PREFILL_KERNEL = "prefill_pipe<0, 32, false>"
DECODE_KERNEL = "decode_kernel<128, 128, linattn::BF16, 0"
PREFILL_PROFILE = "prefill_pipe_delta_B4_H16_T4096_d128.txt"
DECODE_PROFILE = "decode_kernel_delta_N256_H32_d128.txt"
COPY_KERNEL = "copyBuffer"
# (summary file, workload, kernels) of the rows timed by bench_rows: each
# kernel is a name substring, or (substring, grid size in threads) where the
# same kernel runs at several shapes in the traced run
_KDA3 = 4 * 16 * 64   # chunks of the B=4 H=16 T=4096 rows
_KDA4 = 1 * 32 * 512  # chunks of the B=1 H=32 T=32768 rows
ROW_PROFILES = [
    ("prefill_pipe_gated_B1_H32_T32768_d128.txt",
     "gated deltanet_prefill B=1 H=32 T=32768 dk=dv=128 bf16: gate pre-pass + pipelined kernel",
     [("gate_prep<128>", _KDA4 * 256), "prefill_pipe<1, 16, false>"]),
    ("la_par_B8_H12_T1024_d64.txt",
     "la_prefill B=8 H=12 T=1024 dk=dv=64 bf16: chunk states, state scan, chunk outputs",
     ["la_chunk_state<64, 64, false>", "la_state_scan<false>", "la_chunk_out<64, 64, false>"]),
    ("la_par_gla_B8_H12_T1024_d64.txt",
     "gla_prefill B=8 H=12 T=1024 dk=dv=64 bf16: chunk states, decayed state scan, chunk outputs",
     ["la_chunk_state<64, 64, true>", "la_state_scan<true>", "la_chunk_out<64, 64, true>"]),
    ("prefill_pipe_token_gate_B4_H16_T4096_d128.txt",
     "gated_deltanet_prefill (one decay per token) B=4 H=16 T=4096 dk=dv=128 bf16",
     ["prefill_pipe<2, 32, false>"]),
    ("prefill_pipe_token_gate_B1_H32_T32768_d128.txt",
     "gated_deltanet_prefill (one decay per token) B=1 H=32 T=32768 dk=dv=128 bf16",
     ["prefill_pipe<2, 16, false>"]),
    ("prefill_kernel_la_fp32_B1_H2_T64_d16.txt", "la_prefill B=1 H=2 T=64 dk=dv=16 fp32",
     ["prefill_kernel<16, linattn::F32, 0, 16>"]),
    ("decode_kernel_la_N256_H32_d128.txt", "la_decode_step N=256 H=32 dk=dv=128, fp32 S and z",
     ["decode_kernel<128, 128, linattn::BF16, 2"]),
    ("decode_kernel_gated_N256_H32_d128.txt", "gated deltanet_decode_step N=256 H=32 dk=dv=128",
     ["decode_kernel<128, 128, linattn::BF16, 1"]),
    ("decode_kernel_token_gate_N256_H32_d128.txt",
     "gated_deltanet_decode_step (one decay per token) N=256 H=32 dk=dv=128",
     ["decode_kernel<128, 128, linattn::BF16, 3"]),
    ("decode_kernel_gla_N256_H32_d128.txt", "gla_decode_step N=256 H=32 dk=dv=128",
     ["decode_kernel<128, 128, linattn::BF16, 4"]),
    ("delta_backward_B4_H16_T4096_d128.txt",
     "deltanet_prefill_backward B=4 H=16 T=4096 dk=dv=128 bf16: forward chunk states "
     "(pipelined kernel with state capture), transition pre-pass, reverse chain, "
     "chunk-parallel gradients",
     ["prefill_pipe<0, 32, true>", "bwd_transition<128, false, false>",
      "bwd_chain_mat<128, 32, false, false>", "bwd_grads<128, 128, linattn::BF16, false, false>"]),
    ("gated_delta_backward_B4_H16_T4096_d128.txt",
     "gated_deltanet_prefill_backward (one decay per token) B=4 H=16 T=4096 dk=dv=128 bf16: "
     "forward chunk states (pipelined kernel with state capture), transition pre-pass, reverse chain, "
     "chunk-parallel gradients with dg",
     ["prefill_pipe<2, 32, true>", "bwd_transition<128, true, false>",
      "bwd_chain_mat<128, 32, true, false>", "bwd_grads<128, 128, linattn::BF16, true, false>"]),
    ("kda_backward_B4_H16_T4096_d128.txt",
     "kda_prefill_backward (a decay per key channel) B=4 H=16 T=4096 dk=dv=128 bf16: gate "
     "pre-pass, forward chunk states (pipelined kernel with state capture), transition pre-pass, "
     "reverse chain, gradients (dq, dk, dg formed in the same kernel), token walk of "
     "out-of-range chunks (none here: each workgroup exits)",
     [("gate_prep<128>", _KDA3 * 256), "prefill_pipe<1, 32, true>",
      ("bwd_transition<128, false, true>", _KDA3 * 512), ("bwd_chain_mat<128, 32, false, true>", 64 * 4 * 512),
      ("bwd_grads<128, 128, linattn::BF16, false, true>", _KDA3 * 512), ("kda_walk_grads<128, 128>", _KDA3 * 512)]),
    ("kda_backward_B1_H32_T32768_d128.txt",
     "kda_prefill_backward (a decay per key channel) B=1 H=32 T=32768 dk=dv=128 bf16, the gated "
     "workload's decays: the same passes",
     [("gate_prep<128>", _KDA4 * 256), "prefill_pipe<1, 16, true>",
      ("bwd_transition<128, false, true>", _KDA4 * 512), ("bwd_chain_mat<128, 32, false, true>", 32 * 4 * 512),
      ("bwd_grads<128, 128, linattn::BF16, false, true>", _KDA4 * 512), ("kda_walk_grads<128, 128>", _KDA4 * 512)]),
    ("prologue_B4_H16_T4096_d128.txt",
     "deltanet_prologue B=4 H=16 T=4096 dk=128 bf16, one beta logit per token shared by the heads",
     ["qk_prologue<128, linattn::BF16, true>"]),
]


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
    """HBM bytes per launch measured with rocprofv3 counters, if the summary
    in profiles/ was taken on the current kernel source; otherwise None."""
    rec = {}
    try:
        with open(os.path.join(PROFILES, name)) as f:
            for ln in f:
                key, sep, val = ln.partition(":")
                if sep:
                    rec[key.strip()] = val.strip()
    except OSError:
        return None
    if rec.get("kernel_sources_sha256") != digest or "hbm_bytes_per_launch" not in rec:
        return None
    return float(rec["hbm_bytes_per_launch"])


def recorded_counters(name, digest):
    """MFMA and LDS figures per launch from the counter section of a summary
    in profiles/, if it was taken on the current kernel source; else None."""
    rec = {}
    try:
        with open(os.path.join(PROFILES, name)) as f:
            for ln in f:
                key, sep, val = ln.partition(":")
                if sep:
                    rec[key.strip()] = val.split()[0] if val.split() else ""
    except OSError:
        return None
    keys = ("mfma_bf16_flops_per_launch", "mfma_busy_frac", "lds_active_frac",
            "lds_bank_conflict_frac", "effective_clock_ghz")
    if rec.get("kernel_sources_sha256") != digest or any(k not in rec for k in keys):
        return None
    return {k: float(rec[k]) for k in keys}


def _csv_rows(directory, suffix):
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True)):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    return rows


def _counter_mean(directory, counter, kernel):
    vals = [float(r["Counter_Value"]) for r in _csv_rows(directory, "counter_collection.csv")
            if r["Counter_Name"] == counter and kernel in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"no {counter} rows for kernel '{kernel}' under {directory}")
    return sum(vals) / len(vals), len(vals)


PREFILL_SQ_SETS = {
    # one rocprofv3 run each (at most 8 SQ and 2 GRBM counters per run)
    "mfma": ["SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"],
    "lds": ["SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS", "SQ_WAVE_CYCLES"],
}


def _prefill_counter_lines(prof_dir, kname, avg_ns):
    """MFMA and LDS activity of the prefill kernel from two counter runs.
    Counter values are summed over the GPU per dispatch: MFMA busy cycles
    over the 1024 SIMDs, LDS cycles over the 256 CUs, GRBM_GUI_ACTIVE over
    the 8 XCDs (so GRBM / 8 is the kernel's length in cycles)."""
    m = {}
    for tag, counters in PREFILL_SQ_SETS.items():
        for c in counters:
            m[c] = _counter_mean(os.path.join(prof_dir, f"pmc_{tag}_prefill"), c, kname)[0]
    cycles = m["GRBM_GUI_ACTIVE"] / 8.0
    flops = m["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0
    alg_flops = prefill_algorithmic(4, 16, 4096, 128, 128)[1]
    cmd = ("cd /tmp && rocprofv3 --pmc {cs} -f csv -d $OUT/pmc_{t}_prefill -o pmc "
           "-- python3 $R/bench.py --only prefill --steps 5 --warmup 1 --decode-steps 20")
    out = ["", "## MFMA and LDS counters, one run per set"]
    out += [f"#   {cmd.format(cs=' '.join(cs), t=t)}" for t, cs in PREFILL_SQ_SETS.items()]
    out += [f"{c.lower()}_per_dispatch: {m[c]:.0f}" for cs in PREFILL_SQ_SETS.values() for c in cs]
    out += [
        f"kernel_cycles (GRBM_GUI_ACTIVE / 8): {cycles:.0f}",
        f"effective_clock_ghz: {cycles / avg_ns:.3f}   (cycles / traced average ns)",
        f"mfma_bf16_flops_per_launch: {flops:.4g}   (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512)",
        f"algorithmic_flops_per_launch: {alg_flops:.4g}",
        f"executed_over_algorithmic_flops: {flops / alg_flops:.3f}",
        f"mfma_busy_frac: {m['SQ_VALU_MFMA_BUSY_CYCLES'] / (cycles * 1024):.4f}   "
        "(MFMA busy cycles / (kernel cycles x 1024 SIMDs))",
        f"lds_active_frac: {m['SQ_LDS_IDX_ACTIVE'] / (cycles * 256):.4f}   (LDS active cycles / (kernel cycles x 256 CUs))",
        f"lds_bank_conflict_frac: {m['SQ_LDS_BANK_CONFLICT'] / (cycles * 256):.4f}   (of the same)",
    ]
    return out


# Rows whose summaries also carry HBM counters, each from FETCH_SIZE and
# WRITE_SIZE runs of their own (bench.py --only MODE): (summary file, mode,
# kernels of one call, the call's algorithmic bytes).
ROW_COUNTERS = [
    ("prefill_pipe_gated_B1_H32_T32768_d128.txt", "gated-row",
     ["gate_prep<128>", "prefill_pipe<1, 16, false>"], lambda: gated_algorithmic(1, 32, 32768, 128, 128)),
    ("la_par_B8_H12_T1024_d64.txt", "la-rows",
     ["la_chunk_state<64, 64, false>", "la_state_scan<false>", "la_chunk_out<64, 64, false>"],
     lambda: la_algorithmic(8, 12, 1024, 64, 64, 2)),
    ("delta_backward_B4_H16_T4096_d128.txt", "backward-row",
     ["prefill_pipe<0, 32, true>", "bwd_transition<128, false, false>", "bwd_chain_mat<128, 32, false, false>",
      "bwd_grads<128, 128, linattn::BF16, false, false>"],
     lambda: backward_algorithmic(4, 16, 4096, 128, 128)),
]


def _row_counter_lines(prof_dir, mode, kernels, alg, cal):
    """HBM bytes of each kernel of one call (FETCH_SIZE and WRITE_SIZE per
    dispatch, scaled by the copy calibration) and their sum against the
    call's algorithmic bytes."""
    cmd = ("cd /tmp && rocprofv3 --pmc {c} -f csv -d $OUT/pmc_{c}_{m} -o pmc "
           "-- python3 $R/bench.py --only {m}")
    out = ["## HBM counters, one run per counter",
           f"#   {cmd.format(c='FETCH_SIZE', m=mode)}",
           f"#   {cmd.format(c='WRITE_SIZE', m=mode)}",
           f"#   calibration: scale {cal['FETCH_SIZE'][1]:.4f} (fetch), {cal['WRITE_SIZE'][1]:.4f} (write), "
           "from the copy runs of the headline summary"]
    total = 0.0
    for k in kernels:
        f_kib, n = _counter_mean(os.path.join(prof_dir, f"pmc_FETCH_SIZE_{mode}"), "FETCH_SIZE", k)
        w_kib, _ = _counter_mean(os.path.join(prof_dir, f"pmc_WRITE_SIZE_{mode}"), "WRITE_SIZE", k)
        rd = f_kib * 1024.0 * cal["FETCH_SIZE"][1]
        wr = w_kib * 1024.0 * cal["WRITE_SIZE"][1]
        total += rd + wr
        out += [f"counters: {k}   (dispatches {n})",
                f"  hbm_read_bytes_per_launch: {rd:.0f}",
                f"  hbm_write_bytes_per_launch: {wr:.0f}"]
    out += [f"hbm_bytes_per_call: {total:.0f}",
            f"algorithmic_bytes_per_call: {alg}",
            f"traffic_over_algorithmic: {total / alg:.3f}", ""]
    return out


# The segmented row's kernels, from a trace run of its own (the passes run the
# plain pipelined kernel at the grid of the timed prefill, which they would
# otherwise share a summary with).
SEGMENTED_TRACE_CMD = ("cd /tmp && rocprofv3 --kernel-trace --stats -f csv -d "
                       "$OUT/trace_segmented -o trace -- python3 $R/bench.py "
                       "--only segmented-row")
SEGMENTED_PROFILES = [
    ("segmented_B1_H4_T32768_d128.txt",
     "deltanet_prefill_segmented B=1 H=4 T=32768 dk=dv=128 bf16, no gate, 16 segments of 2048 "
     "tokens: start states and zeros, the two passes (pipelined kernel over 64 segment-heads; "
     "value pass and transition pass, two calls each), the scan, the fix-up; and the one-pass "
     "kernel on the same inputs",
     ["seg_prepare", "prefill_pipe<0, 32, false>", "seg_mfrag<128>", "seg_scan<128>",
      "seg_fixup<128, 128>", "prefill_pipe<0, 16, false>"]),
    ("segmented_per_channel_gate_B1_H4_T32768_d128.txt",
     "deltanet_prefill_segmented B=1 H=4 T=32768 dk=dv=128 bf16, a decay per key channel, 16 "
     "segments: the gate pre-pass (once for both passes; the one-pass call runs it too, same "
     "grid), the two gated passes, and the one-pass gated kernel",
     ["gate_prep<128>", "prefill_pipe<1, 32, false>", "prefill_pipe<1, 16, false>"]),
]


def _trace_summaries(dispatches, profiles, trace_cmd):
    """Per-kernel kernel-trace figures (calls, average, min, max) from
    per-dispatch records, one summary file per entry of `profiles`."""
    for fname, wl, kernels in profiles:
        lines = [f"# rocprofv3 kernel-trace summary: {wl}",
                 "# $R is the repository root, $OUT the directory the raw rocprofv3 output goes to; the command runs committed files only.",
                 f"# command: {trace_cmd}", ""]
        for spec in kernels:
            kname, grid = spec if isinstance(spec, tuple) else (spec, None)
            sel = [r for r in dispatches if kname in r["Kernel_Name"]
                   and (grid is None or int(r["Grid_Size_X"]) == grid)]
            names = {r["Kernel_Name"] for r in sel}
            if len(names) != 1:
                raise SystemExit(f"expected one kernel for '{kname}' (grid {grid}), found {len(names)}")
            ns = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in sel]
            lines += [f"kernel: {names.pop()}" + (f"   (grid {grid} threads)" if grid else ""),
                      f"calls: {len(ns)}", f"average_ns: {sum(ns) / len(ns):.0f}",
                      f"min_ns: {min(ns)}", f"max_ns: {max(ns)}", ""]
        with open(os.path.join(PROFILES, fname), "w") as f:
            f.write("\n".join(lines))
        print(f"wrote profiles/{fname}")


def summarize(prof_dir):
    """Write the rocprofv3 summaries in profiles/ from the raw output of the
    profiling commands listed in each summary (run from /tmp, repo at $R):
      trace:  rocprofv3 --kernel-trace --stats -f csv -d $R/<dir>/trace -o trace
                -- python3 $R/bench.py --no-cpu-baseline
      counters, one run per counter C in FETCH_SIZE, WRITE_SIZE and mode M in
      prefill, decode, copy:
              rocprofv3 --pmc C -f csv -d $R/<dir>/pmc_C_M -o pmc
                -- python3 $R/bench.py --only M --steps 5 --warmup 1 --decode-steps 20
    FETCH_SIZE and WRITE_SIZE are in KiB per dispatch; each is scaled by the
    ratio of the true size of a 1 GiB device copy to what the same counter
    reads for it."""
    stats = _csv_rows(os.path.join(prof_dir, "trace"), "kernel_stats.csv")
    copy_bytes = 1 << 30
    cal = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        kib, _ = _counter_mean(os.path.join(prof_dir, f"pmc_{c}_copy"), c, COPY_KERNEL)
        cal[c] = (kib, copy_bytes / (kib * 1024.0))
    trace_cmd = ("cd /tmp && rocprofv3 --kernel-trace --stats -f csv -d $OUT/trace "
                 "-o trace -- python3 $R/bench.py --no-cpu-baseline")
    pmc_cmd = ("cd /tmp && rocprofv3 --pmc {c} -f csv -d $OUT/pmc_{c}_{m} -o pmc "
               "-- python3 $R/bench.py --only {m} --steps 5 --warmup 1 --decode-steps 20")
    jobs = [("prefill", PREFILL_KERNEL, PREFILL_PROFILE, PREFILL_SOURCES,
             "deltanet_prefill B=4 H=16 T=4096 dk=dv=128, bf16 q/k/v/beta/o, fp32 state",
             prefill_algorithmic(4, 16, 4096, 128, 128)[0]),
            ("decode", DECODE_KERNEL, DECODE_PROFILE, DECODE_SOURCES,
             "deltanet_decode_step N=256 H=32 dk=dv=128, fp32 state in place, bf16 token inputs",
             decode_algorithmic(256, 32, 128, 128))]
    for mode, kname, fname, srcs, wl, alg in jobs:
        row = [r for r in stats if kname in r["Name"]]
        if len(row) != 1:
            raise SystemExit(f"expected one kernel-trace row for '{kname}', found {len(row)}")
        row = row[0]
        meas = {}
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            meas[c] = _counter_mean(os.path.join(prof_dir, f"pmc_{c}_{mode}"), c, kname)
        fetch = meas["FETCH_SIZE"][0] * 1024.0 * cal["FETCH_SIZE"][1]
        write = meas["WRITE_SIZE"][0] * 1024.0 * cal["WRITE_SIZE"][1]
        lines = [
            f"# rocprofv3 summary: {row['Name']}",
            f"# workload: {wl}",
            "# $R is the repository root, $OUT the directory the raw rocprofv3 output goes to; every command runs committed files only.",
            f"kernel_sources: {' '.join(srcs)}",
            f"kernel_sources_sha256: {sources_digest(srcs)}",
            "",
            f"## kernel trace  ({trace_cmd})",
            f"calls: {row['Calls']}",
            f"average_ns: {float(row['AverageNs']):.0f}",
            f"min_ns: {float(row['MinNs']):.0f}",
            f"max_ns: {float(row['MaxNs']):.0f}",
            f"stddev_ns: {float(row['StdDev']):.0f}",
            "",
            "## HBM counters, one run per counter",
            f"#   {pmc_cmd.format(c='FETCH_SIZE', m=mode)}",
            f"#   {pmc_cmd.format(c='WRITE_SIZE', m=mode)}",
            f"#   calibration: the same two commands with --only copy ({COPY_KERNEL}, 1 GiB)",
            f"fetch_kib_per_dispatch: {meas['FETCH_SIZE'][0]:.1f}   (dispatches {meas['FETCH_SIZE'][1]})",
            f"write_kib_per_dispatch: {meas['WRITE_SIZE'][0]:.1f}   (dispatches {meas['WRITE_SIZE'][1]})",
            f"copy_fetch_kib: {cal['FETCH_SIZE'][0]:.1f}   scale {cal['FETCH_SIZE'][1]:.4f}",
            f"copy_write_kib: {cal['WRITE_SIZE'][0]:.1f}   scale {cal['WRITE_SIZE'][1]:.4f}",
            f"hbm_read_bytes_per_launch: {fetch:.0f}",
            f"hbm_write_bytes_per_launch: {write:.0f}",
            f"hbm_bytes_per_launch: {fetch + write:.0f}",
            f"algorithmic_bytes_per_launch: {alg}",
            f"traffic_over_algorithmic: {(fetch + write) / alg:.3f}",
        ]
        if mode == "prefill":
            lines += _prefill_counter_lines(prof_dir, kname, float(row["AverageNs"]))
        os.makedirs(PROFILES, exist_ok=True)
        with open(os.path.join(PROFILES, fname), "w") as f:
            f.write("\n".join(lines) + "\n")
        print(f"wrote profiles/{fname}")
    # the other rows: kernel-trace figures only (same trace run), from the
    # per-dispatch records
    _trace_summaries(_csv_rows(os.path.join(prof_dir, "trace"), "kernel_trace.csv"), ROW_PROFILES,
                     trace_cmd)
    for fname, mode, kernels, alg in ROW_COUNTERS:
        if not os.path.isdir(os.path.join(prof_dir, f"pmc_FETCH_SIZE_{mode}")):
            continue
        with open(os.path.join(PROFILES, fname), "a") as f:
            f.write("\n".join(_row_counter_lines(prof_dir, mode, kernels, alg(), cal)))
        print(f"added counters to profiles/{fname}")
    if os.path.isdir(os.path.join(prof_dir, "trace_segmented")):
        _trace_summaries(_csv_rows(os.path.join(prof_dir, "trace_segmented"), "kernel_trace.csv"),
                         SEGMENTED_PROFILES, SEGMENTED_TRACE_CMD)


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


def _time_launches(torch, stream, run, sets, n, warmup=3):
    """Average and median duration of `n` launches of run(set), each between
    its own pair of HIP events on `stream`; the input sets are cycled."""
    for i in range(warmup):
        run(sets[i % len(sets)])
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        run(sets[i % len(sets)])
        b.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return sum(ms) / n * 1e3, ms[n // 2] * 1e3


def _row(name, workload, us, med_us, nbytes, note=None):
    gbs = nbytes / (us * 1e-6) / 1e9
    r = {"workload": workload, "avg_launch_us": us, "median_launch_us": med_us,
         "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": nbytes}}
    if note:
        r["note"] = note
    return name, r


def la_algorithmic(B, H, T, dk, dv, elem_bytes):
    """Bytes a linear-attention prefill must move: q, k, v in and o out, and
    the final state S and normaliser z (fp32)."""
    return B * H * (T * 2 * (dk + dv) * elem_bytes + (dk * dv + dk) * 4)


def backward_algorithmic(B, H, T, dk, dv):
    """Bytes the delta rule's backward must move (bf16): q, k, v, dO and beta
    in; dq, dk, dv and dbeta out."""
    th = B * H * T
    return th * 2 * (2 * dk + 2 * dv + 1) + th * 2 * (2 * dk + dv + 1)


def gated_algorithmic(B, H, T, dk, dv):
    """Bytes the per-channel gated delta-rule prefill must move (bf16): q, k,
    g (one log-decay per key channel), v and beta in, o out, and the final
    fp32 state."""
    return B * H * (T * 2 * (3 * dk + 2 * dv + 1) + dk * dv * 4)


def bench_la_rows(la, workloads, torch, launches=20):
    """The linear-attention prefill rows (fp32 and bf16), each on its own
    workload, with several input copies cycled."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    rows = {}
    W = workloads.WORKLOADS
    for w in (W[0], W[1]):
        inp = workloads.make_workload(w)
        per = la_algorithmic(w.B, w.H, w.T, w.dk, w.dv, 4 if w.dtype == torch.float32 else 2)
        copies = max(1, min(8, -(-600_000_000 // per)))
        sets = []
        for _ in range(copies):
            d = {k: v.to(dev) for k, v in inp.items()}
            d["o"] = torch.empty_like(d["v"])
            d["S"] = torch.empty(w.B, w.H, w.dk, w.dv, device=dev, dtype=torch.float32)
            d["z"] = torch.empty(w.B, w.H, w.dk, device=dev, dtype=torch.float32)
            sets.append(d)

        def run(d):
            la.la_prefill(d["q"], d["k"], d["v"], S=d["S"], z=d["z"], o=d["o"], stream=stream)

        us, med = _time_launches(torch, stream, run, sets, launches)
        name, r = _row("la_prefill", f"la_prefill {w.name}, {copies} input copies cycled",
                       us, med, per,
                       "latency-bound: one 64-token chunk" if w.T == 64 else None)
        rows[f"{name}_{w.name}"] = r
        del sets
    return rows


def bench_gated_row(la, workloads, torch, launches=20):
    """The per-channel gated delta-rule prefill on the gated workload."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    w = workloads.WORKLOADS[3]
    inp = workloads.make_workload(w)
    d = {k: v.to(dev) for k, v in inp.items()}
    d["o"] = torch.empty_like(d["v"])
    d["S"] = torch.empty(w.B, w.H, w.dk, w.dv, device=dev, dtype=torch.float32)
    del inp

    def run_g(d):
        la.deltanet_prefill(d["q"], d["k"], d["v"], d["beta"], g=d["g"], S=d["S"], o=d["o"],
                            stream=stream)

    us, med = _time_launches(torch, stream, run_g, [d], max(3, launches // 4), warmup=1)
    per = gated_algorithmic(w.B, w.H, w.T, w.dk, w.dv)
    name, r = _row("deltanet_prefill_gated", f"deltanet_prefill (gated) {w.name}", us, med, per,
                   "gate pre-pass, then a serial chain over 512 chunks; 32 heads x 8 value "
                   "slices of 16 = 256 workgroups")
    return {name: r}


def bench_rows(la, workloads, torch, launches=20):
    """The remaining rows of the path, each timed on its own workload: linear
    attention prefill (fp32 and bf16), the gated delta-rule prefill, and the
    linear-attention and gated decode steps at the decode workload's shape."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    rows = bench_la_rows(la, workloads, torch, launches)
    rows.update(bench_gated_row(la, workloads, torch, launches))
    wd = workloads.WORKLOADS[4]
    N, H, dk, dv = wd.B, wd.H, wd.dk, wd.dv
    li = workloads.make_la_decode(N, H, dk, dv, wd.dtype, seed=77)
    d = {k: v.to(dev) for k, v in li.items()}
    o = torch.empty(N, H, dv, device=dev, dtype=wd.dtype)
    ring = d["q"].shape[0]
    cnt = [0]

    def run_ld(_):
        s = cnt[0] % ring
        cnt[0] += 1
        la.la_decode_step(d["q"][s], d["k"][s], d["v"][s], d["S0"], d["z0"], o=o, stream=stream)

    us, med = _time_launches(torch, stream, run_ld, [None], 200, warmup=10)
    per = N * H * (2 * (dk * dv + dk) * 4 + 2 * (2 * dk + 2 * dv))
    name, r = _row("la_decode_step", f"la_decode_step N={N} H={H} dk=dv={dk}, fp32 S and z "
                   "in place", us, med, per)
    rows[name] = r
    del d, li
    gi = workloads.make_decode(N, H, dk, dv, wd.dtype, seed=78, gated=True)
    d = {k: v.to(dev) for k, v in gi.items()}
    cnt[0] = 0

    def run_gd(_):
        s = cnt[0] % ring
        cnt[0] += 1
        la.deltanet_decode_step(d["q"][s], d["k"][s], d["v"][s], d["beta"][s], d["S0"],
                                g=d["g"][s], o=o, stream=stream)

    us, med = _time_launches(torch, stream, run_gd, [None], 200, warmup=10)
    per = N * H * (2 * dk * dv * 4 + 2 * (3 * dk + 2 * dv + 1))
    name, r = _row("deltanet_decode_step_gated", f"deltanet_decode_step (gated) N={N} H={H} "
                   f"dk=dv={dk}, fp32 state in place", us, med, per)
    rows[name] = r
    del d, gi
    rows.update(bench_token_gated_rows(la, workloads, torch, launches))
    rows.update(bench_backward_row(la, workloads, torch))
    rows.update(bench_prologue_row(la, workloads, torch))
    return rows


def bench_prologue_row(la, workloads, torch, launches=20):
    """The layer prologue (q, k = normalize(silu(.)), beta = sigmoid of one
    logit per token) at the timed prefill workload's shape."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    w = workloads.WORKLOADS[2]
    gen = workloads.generator(97)
    q = torch.randn(w.B, w.H, w.T, w.dk, generator=gen).to(w.dtype).to(dev)
    k = torch.randn(w.B, w.H, w.T, w.dk, generator=gen).to(w.dtype).to(dev)
    lg = torch.randn(w.B, 1, w.T, generator=gen).to(w.dtype).to(dev)
    qo, ko = torch.empty_like(q), torch.empty_like(k)

    def run(_):
        la.deltanet_prologue(q, k, lg, out=(qo, ko), stream=stream)

    us, med = _time_launches(torch, stream, run, [None], launches)
    th = w.B * w.H * w.T
    per = th * 2 * 2 * w.dk * 2 + w.B * w.T * 2 + th * 2
    name, r = _row("deltanet_prologue", f"deltanet_prologue B={w.B} H={w.H} T={w.T} dk={w.dk} "
                   "bf16, beta shared by the heads", us, med, per)
    return {name: r}


def bench_backward_row(la, workloads, torch, launches=5):
    """The delta rule's gradient at the timed prefill workload's shape: the
    forward chunk states, the reverse chain and the chunk-parallel gradients."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    w = workloads.WORKLOADS[2]
    inp = workloads.make_delta(w.B, w.H, w.T, w.dk, w.dv, w.dtype, seed=95)
    d = {k: v.to(dev) for k, v in inp.items()}
    gen = workloads.generator(96)
    d["dO"] = torch.randn(w.B, w.H, w.T, w.dv, generator=gen).to(w.dtype).to(dev)
    del inp

    def run(d):
        la.deltanet_prefill_backward(d["q"], d["k"], d["v"], d["beta"], d["dO"], stream=stream)

    us, med = _time_launches(torch, stream, run, [d], launches, warmup=1)
    th = w.B * w.H * w.T
    per = backward_algorithmic(w.B, w.H, w.T, w.dk, w.dv)
    name, r = _row("deltanet_prefill_backward", f"deltanet_prefill_backward B={w.B} H={w.H} "
                   f"T={w.T} dk=dv={w.dk} bf16", us, med, per,
                   "four kernels: forward chunk states (pipelined kernel, states captured), "
                   "chunk-parallel transition pre-pass (P = W^T K, R = Q - A W), reverse chain "
                   "dS <- dS - P dS + R^T dO, chunk-parallel gradients; bytes are the inputs "
                   "(q, k, v, beta, dO) and gradients (dq, dk, dv, dbeta) only")
    rows = {name: r}
    gen = workloads.generator(98)
    d["g"] = (-torch.nn.functional.softplus(torch.randn(w.B, w.H, w.T, generator=gen)) / 16.0
              ).to(w.dtype).to(dev)

    def run_g(d):
        la.gated_deltanet_prefill_backward(d["q"], d["k"], d["v"], d["beta"], d["g"], d["dO"],
                                           stream=stream)

    us, med = _time_launches(torch, stream, run_g, [d], launches, warmup=1)
    name, r = _row("gated_deltanet_prefill_backward", "gated_deltanet_prefill_backward (one decay "
                   f"per token) B={w.B} H={w.H} T={w.T} dk=dv={w.dk} bf16", us, med,
                   per + 2 * th * 2,
                   "four kernels: forward chunk states (pipelined kernel, states captured), "
                   "transition pre-pass with the decays, reverse chain with the chunk decay, "
                   "chunk-parallel gradients and dg; bytes as above plus g in and dg out")
    rows[name] = r
    # a decay per key channel, at the timed shape and at the gated workload's
    for wk, seed in ((w, 99), (workloads.WORKLOADS[3], 100)):
        if wk is not w:
            inp = workloads.make_workload(wk)
            d = {k: v.to(dev) for k, v in inp.items() if k != "S0"}
            del inp
            gen = workloads.generator(seed)
            d["dO"] = torch.randn(wk.B, wk.H, wk.T, wk.dv, generator=gen).to(wk.dtype).to(dev)
        else:
            gen = workloads.generator(seed)
            d["g"] = (-torch.nn.functional.softplus(torch.randn(w.B, w.H, w.T, w.dk, generator=gen))
                      / 16.0).to(w.dtype).to(dev)
        ws = torch.empty(la.kda_prefill_backward_workspace_bytes(wk.B, wk.H, wk.T, wk.dk, wk.dv,
                                                                 wk.dtype),
                         device=dev, dtype=torch.uint8)

        def run_k(d):
            la.kda_prefill_backward(d["q"], d["k"], d["v"], d["beta"], d["g"], d["dO"],
                                    stream=stream, workspace=ws)

        us, med = _time_launches(torch, stream, run_k, [d], launches, warmup=1)
        thk = wk.B * wk.H * wk.T
        perk = (thk * 2 * (2 * wk.dk + 2 * wk.dv + 1) + thk * 2 * (2 * wk.dk + wk.dv + 1)
                + 2 * thk * 2 * wk.dk)
        name, r = _row("kda_prefill_backward", "kda_prefill_backward (a decay per key channel) "
                       f"B={wk.B} H={wk.H} T={wk.T} dk=dv={wk.dk} bf16", us, med, perk,
                       "six kernels: gate pre-pass, forward chunk states (pipelined kernel on "
                       "the pre-pass's tiles, states captured), transition pre-pass, reverse "
                       "chain with the per-channel chunk decay, chunk-parallel gradients (dq, "
                       "dk, dg included), the out-of-range chunks' token walk (none here); "
                       "bytes as the other backward rows plus g in and dg out [B,H,T,dk]")
        rows[f"{name}_T{wk.T}"] = r
        del ws
    return rows


def bench_token_gated_rows(la, workloads, torch, launches=20):
    """The per-token gated entry points: the Gated DeltaNet prefill at the
    delta-rule and gated workloads' shapes, gated linear attention at the
    bf16 linear-attention workload's shape, and both decode steps at the
    decode workload's shape."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    rows = {}
    W = workloads.WORKLOADS
    for w in (W[2], W[3]):
        inp = workloads.make_delta(w.B, w.H, w.T, w.dk, w.dv, w.dtype, seed=90 + w.index,
                                   gated="token")
        d = {k: v.to(dev) for k, v in inp.items()}
        d["o"] = torch.empty_like(d["v"])
        d["S"] = torch.empty(w.B, w.H, w.dk, w.dv, device=dev, dtype=torch.float32)
        del inp

        def run(d):
            la.gated_deltanet_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], S=d["S"],
                                      o=d["o"], stream=stream)

        us, med = _time_launches(torch, stream, run, [d], max(5, launches // 2), warmup=2)
        per = w.B * w.H * (w.T * 2 * (2 * w.dk + 2 * w.dv + 2) + w.dk * w.dv * 4)
        name, r = _row("gated_deltanet_prefill", f"gated_deltanet_prefill (one decay per token) "
                       f"B={w.B} H={w.H} T={w.T} dk=dv={w.dk} bf16", us, med, per)
        rows[f"{name}_T{w.T}"] = r
        del d
    w = W[1]
    inp = workloads.make_gla(w.B, w.H, w.T, w.dk, w.dv, w.dtype, seed=92)
    d = {k: v.to(dev) for k, v in inp.items()}
    d["o"] = torch.empty_like(d["v"])
    d["S"] = torch.empty(w.B, w.H, w.dk, w.dv, device=dev, dtype=torch.float32)

    def run_gla(d):
        la.gla_prefill(d["q"], d["k"], d["v"], d["g"], S=d["S"], o=d["o"], stream=stream)

    us, med = _time_launches(torch, stream, run_gla, [d], launches)
    per = w.B * w.H * (w.T * 2 * (2 * w.dk + 2 * w.dv + 1) + w.dk * w.dv * 4)
    name, r = _row("gla_prefill", f"gla_prefill B={w.B} H={w.H} T={w.T} dk=dv={w.dk} bf16",
                   us, med, per)
    rows[name] = r
    del d, inp
    wd = W[4]
    N, H, dk, dv = wd.B, wd.H, wd.dk, wd.dv
    gi = workloads.make_decode(N, H, dk, dv, wd.dtype, seed=93, gated="token")
    d = {k: v.to(dev) for k, v in gi.items()}
    o = torch.empty(N, H, dv, device=dev, dtype=wd.dtype)
    ring = d["q"].shape[0]
    cnt = [0]

    def run_gd(_):
        s = cnt[0] % ring
        cnt[0] += 1
        la.gated_deltanet_decode_step(d["q"][s], d["k"][s], d["v"][s], d["beta"][s], d["g"][s],
                                      d["S0"], o=o, stream=stream)

    us, med = _time_launches(torch, stream, run_gd, [None], 200, warmup=10)
    per = N * H * (2 * dk * dv * 4 + 2 * (2 * dk + 2 * dv + 2))
    name, r = _row("gated_deltanet_decode_step", f"gated_deltanet_decode_step N={N} H={H} "
                   f"dk=dv={dk}, fp32 state in place", us, med, per)
    rows[name] = r
    cnt[0] = 0

    def run_gld(_):
        s = cnt[0] % ring
        cnt[0] += 1
        la.gla_decode_step(d["q"][s], d["k"][s], d["v"][s], d["S0"], g=d["g"][s], o=o,
                           stream=stream)

    us, med = _time_launches(torch, stream, run_gld, [None], 200, warmup=10)
    per = N * H * (2 * dk * dv * 4 + 2 * (2 * dk + 2 * dv + 1))
    name, r = _row("gla_decode_step", f"gla_decode_step N={N} H={H} dk=dv={dk}, fp32 state "
                   "in place", us, med, per)
    rows[name] = r
    return rows


def bench_segmented_row(la, workloads, torch, launches=20):
    """deltanet_prefill_segmented at the shape it is for, B=1 H=4 T=32768
    d=128 (the automatic count: 16 segments of 2048 tokens), without a gate
    and with a decay per key channel, next to the one-pass entry point on the
    same inputs.  The roofline figure uses the operation's algorithmic bytes
    (those of the one-pass prefill): the segmented call moves more, but the
    row reports what the caller gets.  Timed by HIP events around each call
    on the stream the kernels run on; profiled on its own (the passes run the
    plain pipelined kernel at the grid of the timed prefill)."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    B, H, T, d = 1, 4, 32768, 128
    P = la.deltanet_prefill_segments(B, H, T, d, d)
    nbytes, _ = prefill_algorithmic(B, H, T, d, d)
    rows = {}
    for name, gate in (("segmented_no_gate", None), ("segmented_per_channel_gate", "channel")):
        gen = {None: False, "channel": True}[gate]
        sets = []
        for s in range(2):
            inp = workloads.make_delta(B, H, T, d, d, torch.bfloat16, seed=90 + s, gated=gen)
            sets.append({k: v.to(dev) for k, v in inp.items()})
        o = torch.empty_like(sets[0]["v"])
        S = torch.empty(B, H, d, d, device=dev, dtype=torch.float32)
        ws1 = torch.empty(max(la.deltanet_prefill_workspace_bytes(gate is not None, B, H, T, d, d,
                                                                  torch.bfloat16), 1),
                          device=dev, dtype=torch.uint8)
        ws = torch.empty(la.deltanet_prefill_segmented_workspace_bytes(gate, B, H, T, d, d,
                                                                        torch.bfloat16, P),
                         device=dev, dtype=torch.uint8)

        def one(x):
            la.deltanet_prefill(x["q"], x["k"], x["v"], x["beta"], g=x.get("g"), S=S, o=o,
                                stream=stream, workspace=ws1)

        def seg(x):
            la.deltanet_prefill_segmented(x["q"], x["k"], x["v"], x["beta"], g=x.get("g"), gate=gate,
                                          S=S, o=o, segments=P, stream=stream, workspace=ws)

        us1, med1 = _time_launches(torch, stream, one, sets, launches)
        us, med = _time_launches(torch, stream, seg, sets, launches)
        wl = (f"deltanet_prefill_segmented B={B} H={H} T={T} dk=dv={d} bf16, {P} segments"
              + (", a decay per key channel" if gate else ""))
        _, r = _row(name, wl, us, med, nbytes)
        r["segments"] = P
        r["one_pass_avg_launch_us"] = us1
        r["one_pass_median_launch_us"] = med1
        r["speedup_over_one_pass"] = us1 / us
        rows[name] = r
        del sets, o, S, ws, ws1
        torch.cuda.empty_cache()
    return rows


def bench_segmented_rows(la, workloads, torch, launches=10):
    """deltanet_prefill_segmented (the sequence-parallel chunk-state scan)
    against the one-pass prefill at the same shape: few heads with a long
    sequence (B=1, H=4/8/16, T=32768, d=128; no gate, a decay per key
    channel, one decay per token), where it is meant to win, and the gated
    workload's shape (B=1 H=32 T=32768), where the automatic count declines
    it.  Each entry: the one-pass time and, per segment count, the segmented
    time per call (HIP events around the whole call on the stream the kernels
    run on), the speedup, and the difference from the one-pass result."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    T, d = 32768, 128
    cases = [("no_gate_B1_H4_T32768", 4, None, (0, 4, 8, 16, 32)),
             ("per_channel_gate_B1_H4_T32768", 4, "channel", (0, 8, 16)),
             ("per_token_gate_B1_H4_T32768", 4, "token", (0, 8, 16)),
             ("no_gate_B1_H8_T32768", 8, None, (0, 4, 16)),
             ("no_gate_B1_H16_T32768", 16, None, (0, 2, 8)),
             ("per_channel_gate_B1_H32_T32768", 32, "channel", (0, 2, 4))]
    out = {}
    for name, H, gate, seg_counts in cases:
        gen = {None: False, "channel": True, "token": "token"}[gate]
        inp = workloads.make_delta(1, H, T, d, d, torch.bfloat16, seed=70 + H, gated=gen)
        x = {k: v.to(dev) for k, v in inp.items()}
        del inp
        g = x.get("g")
        o1 = torch.empty_like(x["v"])
        S1 = torch.empty(1, H, d, d, device=dev, dtype=torch.float32)
        ws1 = torch.empty(max(la.deltanet_prefill_workspace_bytes(gate == "channel", 1, H, T, d, d,
                                                                  torch.bfloat16), 1),
                          device=dev, dtype=torch.uint8)

        def one_pass(_):
            if gate == "token":
                la.gated_deltanet_prefill(x["q"], x["k"], x["v"], x["beta"], g, S=S1, o=o1,
                                          stream=stream)
            else:
                la.deltanet_prefill(x["q"], x["k"], x["v"], x["beta"], g=g, S=S1, o=o1,
                                    stream=stream, workspace=ws1)

        us1, _ = _time_launches(torch, stream, one_pass, [None], launches, warmup=2)
        one_pass(None)
        entry = {"one_pass_us": us1, "auto_segments": la.deltanet_prefill_segments(1, H, T, d, d),
                 "segmented": {}}
        o2 = torch.empty_like(o1)
        S2 = torch.empty_like(S1)
        for P in seg_counts:
            ws = torch.empty(max(la.deltanet_prefill_segmented_workspace_bytes(
                gate, 1, H, T, d, d, torch.bfloat16, P), 1), device=dev, dtype=torch.uint8)

            def seg(_):
                la.deltanet_prefill_segmented(x["q"], x["k"], x["v"], x["beta"], g=g, gate=gate,
                                              S=S2, o=o2, segments=P, stream=stream, workspace=ws)

            us, _ = _time_launches(torch, stream, seg, [None], launches, warmup=2)
            seg(None)
            torch.cuda.synchronize()
            o_diff = ((o2.float() - o1.float()).abs().max() / o1.float().abs().max()).item()
            s_diff = ((S2 - S1).abs().max() / S1.abs().max()).item()
            key = f"P{P}" if P else f"auto(P{entry['auto_segments']})"
            entry["segmented"][key] = {"us": us, "speedup": us1 / us, "o_rel_diff": o_diff,
                                       "S_rel_diff": s_diff}
            del ws
        out[name] = entry
        del x, o1, S1, o2, S2, ws1
        torch.cuda.empty_cache()
    return out


def measured_peaks(torch, reps=5):
    """Rates this GPU sustains in the same run, from libpeak_probe.so (built
    with the library): a copy between two buffers (the prefill's pattern:
    inputs read, outputs written elsewhere) and an in-place update (the
    decode's pattern), both averaged over back-to-back launches, and a dense
    bf16 MFMA loop (32x32x16 tiles; random operands draw more power than
    zeros, and the clock follows), best of `reps` launches."""
    import ctypes
    path = os.path.join(ROOT, "delta_rule_recurrent_chunkwise_amd", "libpeak_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m delta_rule_recurrent_chunkwise_amd.build`")
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    lib.peak_probe_mfma_bf16.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, vp]
    lib.peak_probe_stream.argtypes = [vp, vp, ctypes.c_size_t, ctypes.c_int, vp]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = vp(stream.cuda_stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def best_ms(launch):
        best = None
        for _ in range(reps + 1):  # the first launch is a warm-up
            ev[0].record(stream)
            rc = launch()
            ev[1].record(stream)
            ev[1].synchronize()
            if rc != 0:
                raise RuntimeError(f"peak probe returned {rc}")
            ms = ev[0].elapsed_time(ev[1])
            best = ms if best is None else min(best, ms)
        return best

    def avg_ms(launch, n=20):
        for _ in range(3):
            launch()
        ev[0].record(stream)
        for _ in range(n):
            if launch() != 0:
                raise RuntimeError("peak probe launch failed")
        ev[1].record(stream)
        ev[1].synchronize()
        return ev[0].elapsed_time(ev[1]) / n

    nbytes = 512 << 20  # the decode state's size, above the 256 MB Infinity Cache
    src = torch.ones(nbytes // 4, device=dev, dtype=torch.float32)
    dst = torch.empty_like(src)
    copy_gbs = 2 * nbytes / (avg_ms(lambda: lib.peak_probe_stream(src.data_ptr(), dst.data_ptr(), nbytes, 0, sp)) * 1e-3) / 1e9
    rmw_gbs = 2 * nbytes / (avg_ms(lambda: lib.peak_probe_stream(src.data_ptr(), None, nbytes, 1, sp)) * 1e-3) / 1e9
    del src, dst
    blocks, iters = 256 * 4, 4000
    seed = torch.rand(64, device=dev, dtype=torch.float32)
    sink = torch.empty(blocks * 256, device=dev, dtype=torch.float32)
    ms = best_ms(lambda: lib.peak_probe_mfma_bf16(seed.data_ptr(), sink.data_ptr(), blocks, iters, sp))
    mfma_tflops = blocks * 4 * iters * 4 * 32768 / (ms * 1e-3) / 1e12
    return {"copy_gbs": copy_gbs, "in_place_gbs": rmw_gbs, "mfma_bf16_tflops": mfma_tflops,
            "note": "measured before the timed work (libpeak_probe.so): a 512 MiB copy between two "
                    "buffers and a 512 MiB in-place update, 20 back-to-back launches each (read + "
                    "write bytes); a dense 32x32x16 bf16 MFMA loop on random operands, best of 5"}


def copy_probe(torch, nbytes=1 << 30, reps=5):
    """A plain device copy of known size (used to calibrate HBM counters)."""
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, device=dev, dtype=torch.float32)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return nbytes


def host_cores():
    """The host cores this process may use: its CPU affinity, capped by
    OMP_NUM_THREADS where the environment sets it (a shared multi-GPU host
    gives each GPU's job a share of its cores and says so there, whatever
    the affinity mask shows)."""
    n = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS")
    if share and share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return n


def parity_leg(la, workloads, oracle, torch):
    """The oracle's results against the GPU's for every workload, as the
    bench line's record of the achieved error: max|gpu - ref| / max|ref| of
    o, S (and z) over whole tensors for the four prefill workloads, and for
    the decode workload over the full state and every output after one
    step."""
    dev = torch.device("cuda:0")

    def err(gpu, ref):
        import numpy as np
        g = gpu.detach().to("cpu", torch.float64).numpy()
        r = np.asarray(ref, np.float64)
        if not np.all(np.isfinite(g)):
            return float("inf")
        return float(np.max(np.abs(g - r)) / max(float(np.max(np.abs(r))), 1e-300))

    out = {}
    for w in workloads.WORKLOADS:
        inp = workloads.make_workload(w)
        d = {n: t.to(dev) for n, t in inp.items()}
        tol = 1e-4 if w.dtype == torch.float32 else 2e-2
        if w.kind == "la":
            o, S, z = la.la_prefill(d["q"], d["k"], d["v"])
            torch.cuda.synchronize()
            ro, rS, rz = oracle.la_recurrent(inp["q"], inp["k"], inp["v"])
            e = {"o": err(o, ro), "S": err(S, rS), "z": err(z, rz)}
        elif w.kind in ("delta", "gated"):
            o, S = la.deltanet_prefill(d["q"], d["k"], d["v"], d["beta"], g=d.get("g"))
            torch.cuda.synchronize()
            del d
            ro, rS = oracle.delta_recurrent(inp["q"], inp["k"], inp["v"], inp["beta"],
                                            inp.get("g"))
            e = {"o": err(o, ro), "S": err(S, rS)}
        else:
            S = d["S0"].clone()
            o = la.deltanet_decode_step(d["q"][0], d["k"][0], d["v"][0], d["beta"][0], S)
            torch.cuda.synchronize()
            ro, rS = oracle.delta_recurrent(inp["q"][0][:, :, None], inp["k"][0][:, :, None],
                                            inp["v"][0][:, :, None],
                                            inp["beta"][0][:, :, None], None, S0=inp["S0"])
            e = {"o step 1": err(o, ro[:, :, 0]), "S step 1": err(S, rS)}
        e["tol"] = tol
        e["ok"] = all(v <= tol for k, v in e.items() if k != "tol")
        out[w.name] = e
        del inp
    return out


def cpu_baseline(workloads, oracle, torch, prefill_inp, w, decode_inp, wd, budget_s=10.0,
                 decode_budget_s=3.0):
    """The float64 oracle (as written, untuned) timed on the host cores: whole
    passes over the prefill workload, repeated until about `budget_s` seconds
    of work are done, and whole decode steps over all heads for about
    `decode_budget_s` seconds."""
    cores = host_cores()
    x = {n: prefill_inp[n].contiguous() for n in ("q", "k", "v", "beta")}
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.delta_recurrent(x["q"], x["k"], x["v"], x["beta"], nthreads=cores)
        passes += 1
        el = time.perf_counter() - t0
        if el > budget_s:
            break
    tok_s = passes * w.B * w.T / el
    q = decode_inp
    dq = {n: q[n][0][:, :, None].contiguous() for n in ("q", "k", "v", "beta")}
    steps = 0
    t1 = time.perf_counter()
    while True:
        oracle.delta_recurrent(dq["q"], dq["k"], dq["v"], dq["beta"], None, S0=q["S0"],
                               nthreads=cores)
        steps += 1
        el_d = time.perf_counter() - t1
        if el_d > decode_budget_s:
            break
    dec_bytes = decode_algorithmic(wd.B, wd.H, wd.dk, wd.dv)
    return {
        "value": tok_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
        "sample": (f"float64 per-token recurrence, {passes} whole passes over the prefill "
                   f"workload (B={w.B}, H={w.H}, T={w.T}, d={w.dk}) in {el:.1f} s "
                   f"on {cores} threads"),
        "decode": {"value": dec_bytes * steps / el_d / 1e9, "unit": "GB/s",
                   "sample": (f"{steps} decode steps over all {wd.B * wd.H} heads "
                              f"(float64 state) in {el_d:.1f} s")},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the other rows (LA prefill, gated prefill, LA/gated decode)")
    ap.add_argument("--only", choices=["all", "prefill", "decode", "copy", "rows", "token-rows",
                                       "backward-row", "prologue-row", "segmented",
                                       "segmented-row", "la-rows", "gated-row"],
                    default="all",
                    help="run one part only (for profiler runs)")
    ap.add_argument("--summarize", metavar="DIR",
                    help="write profiles/*.txt from rocprofv3 output under DIR and exit")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize)
        return
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
    if args.only == "rows":
        print(json.dumps(bench_rows(la, workloads, torch)))
        return
    if args.only == "la-rows":
        print(json.dumps(bench_la_rows(la, workloads, torch)))
        return
    if args.only == "gated-row":
        print(json.dumps(bench_gated_row(la, workloads, torch)))
        return
    if args.only == "token-rows":
        print(json.dumps(bench_token_gated_rows(la, workloads, torch)))
        return
    if args.only == "backward-row":
        print(json.dumps(bench_backward_row(la, workloads, torch)))
        return
    if args.only == "prologue-row":
        print(json.dumps(bench_prologue_row(la, workloads, torch)))
        return
    if args.only == "segmented":
        print(json.dumps(bench_segmented_rows(la, workloads, torch)))
        return
    if args.only == "segmented-row":
        print(json.dumps(bench_segmented_row(la, workloads, torch)))
        return
    if args.only == "decode":
        wd, _, el = bench_decode(la, workloads, torch, args.decode_steps)
        print(json.dumps({"decode_us_per_step": el / args.decode_steps * 1e6}))
        return

    # peak rates first, while the GPU is still cool (clocks drop under the
    # sustained load that follows)
    peaks = measured_peaks(torch) if args.only == "all" else None
    w, pinp, wall, kms = bench_prefill(la, workloads, torch, args.steps, args.warmup)
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    ms_per_step = wall / args.steps * 1e3
    avg_kernel_s = sum(kms) / len(kms) / 1e3
    pbytes, pflops = prefill_algorithmic(B, H, T, dk, dv)
    achieved = pbytes / avg_kernel_s / 1e9
    traffic = recorded_traffic(PREFILL_PROFILE, sources_digest(PREFILL_SOURCES))
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
                     "kernel": PREFILL_KERNEL,
                     "algorithmic_bytes_per_launch": pbytes,
                     "avg_launch_us": avg_kernel_s * 1e6,
                     "median_launch_us": kms[len(kms) // 2] * 1e3,
                     "min_launch_us": kms[0] * 1e3},
        "mfma": {"achieved": pflops / avg_kernel_s / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                 "unit": "TFLOP/s", "frac": pflops / avg_kernel_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                 "algorithmic_flops_per_launch": pflops,
                 "counters": recorded_counters(PREFILL_PROFILE, sources_digest(PREFILL_SOURCES))},
    }
    if peaks is not None:
        line["measured_peaks"] = peaks
        line["roofline"]["frac_of_measured_copy"] = achieved / peaks["copy_gbs"]
        line["mfma"]["frac_of_measured_peak"] = line["mfma"]["achieved"] / peaks["mfma_bf16_tflops"]
    dinp = None
    if args.only == "all":
        wd, dinp, el = bench_decode(la, workloads, torch, args.decode_steps)
        dbytes = decode_algorithmic(wd.B, wd.H, wd.dk, wd.dv)
        gbs = dbytes * args.decode_steps / el / 1e9
        dtraffic = recorded_traffic(DECODE_PROFILE, sources_digest(DECODE_SOURCES))
        line["decode"] = {
            "value": gbs, "unit": "GB/s", "steps": args.decode_steps, "warmup": 10,
            "us_per_step": el / args.decode_steps * 1e6,
            "config": {"workload": f"deltanet_decode_step N={wd.B} H={wd.H} dk=dv={wd.dk}, "
                                   "fp32 state in place, bf16 token inputs (ring of 16)"},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": dtraffic,
                         "frac_of_measured_in_place": gbs / peaks["in_place_gbs"],
                         "kernel": "decode_kernel<128, 128, BF16, DEC_DELTA>",
                         "avg_launch_us": el / args.decode_steps * 1e6,
                         "algorithmic_bytes_per_launch": dbytes},
        }
        if not args.no_rows:
            line["rows"] = bench_rows(la, workloads, torch)
        if not args.no_cpu_baseline:
            # the CPU leg: the oracle, timed as the baseline, and its results
            # against the GPU's for every workload
            import oracle
            line["cpu_baseline"] = cpu_baseline(workloads, oracle, torch, pinp, w, dinp, wd)
            line["parity"] = parity_leg(la, workloads, oracle, torch)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
