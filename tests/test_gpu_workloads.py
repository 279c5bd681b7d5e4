"""The five workloads at full size, in the launch configuration bench.py
times, against the float64 oracle: full tensors for the prefills; for the
decode workload the full state after step 1 and sampled (sequence, head)
pairs after all 1010 steps.  The backward rows, whose oracle is a slower
reverse recurrence, are compared on sampled heads, which the oracle
recomputes independently (heads never interact)."""
import numpy as np
import pytest
import torch

import delta_rule_recurrent_chunkwise_amd as la
import oracle
import workloads
from gpu_common import TOL, assert_close, require_gpu

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS


def _to(d, dev):
    return {k: v.to(dev) for k, v in d.items()}


@pytest.mark.parametrize("w", [W[0], W[1]], ids=lambda w: w.name)
def test_la_workload_full(w):
    dev = require_gpu()
    print(f"workload {w.name}", flush=True)
    inp = workloads.make_workload(w)
    d = _to(inp, dev)
    o, S, z = la.la_prefill(d["q"], d["k"], d["v"])
    torch.cuda.synchronize()
    o_ref, S_ref, z_ref = oracle.la_recurrent(inp["q"], inp["k"], inp["v"])
    tol = TOL[w.dtype]
    assert_close(o, o_ref, tol, "o")
    assert_close(S, S_ref, tol, "S")
    assert_close(z, z_ref, tol, "z")


def test_deltanet_workload_full():
    dev = require_gpu()
    w = W[2]
    print(f"workload {w.name}", flush=True)
    inp = workloads.make_workload(w)
    d = _to(inp, dev)
    o, S = la.deltanet_prefill(d["q"], d["k"], d["v"], d["beta"])
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.delta_recurrent(inp["q"], inp["k"], inp["v"], inp["beta"])
    assert_close(o, o_ref, TOL[w.dtype], "o")
    assert_close(S, S_ref, TOL[w.dtype], "S")


def test_gated_workload_full():
    """The per-key-channel gated workload (B=1 H=32 T=32768 d=128 bf16) on
    every head: o and the final state against the oracle's full recurrence."""
    dev = require_gpu()
    w = W[3]
    print(f"workload {w.name}", flush=True)
    inp = workloads.make_workload(w)
    d = _to(inp, dev)
    o, S = la.deltanet_prefill(d["q"], d["k"], d["v"], d["beta"], g=d["g"])
    torch.cuda.synchronize()
    del d
    o_ref, S_ref = oracle.delta_recurrent(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"])
    assert_close(o, o_ref, TOL[w.dtype], "o (all heads)")
    assert_close(S, S_ref, TOL[w.dtype], "S (all heads)")


def test_decode_workload():
    """Step 1 on the full 512 MiB state; then 10 + 1000 consecutive steps (the
    bench's warm-up and timed steps, ring slot i mod 16) compared on 64 sampled
    (sequence, head) pairs replayed by the oracle."""
    dev = require_gpu()
    w = W[4]
    print(f"workload {w.name}", flush=True)
    inp = workloads.make_workload(w)
    ring = inp["q"].shape[0]
    d = _to(inp, dev)
    S = d["S0"].clone()
    o = la.deltanet_decode_step(d["q"][0], d["k"][0], d["v"][0], d["beta"][0], S)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.delta_recurrent(inp["q"][0][:, :, None], inp["k"][0][:, :, None],
                                          inp["v"][0][:, :, None],
                                          inp["beta"][0][:, :, None], None, S0=inp["S0"])
    assert_close(o, o_ref[:, :, 0], TOL[w.dtype], "o step 1")
    assert_close(S, S_ref, TOL[w.dtype], "S step 1 (full state)")
    del S_ref
    steps = 1010
    for i in range(1, steps):
        s = i % ring
        o = la.deltanet_decode_step(d["q"][s], d["k"][s], d["v"][s], d["beta"][s], S)
    torch.cuda.synchronize()
    gen = np.random.default_rng(0)
    pairs = sorted(set(zip(gen.integers(0, w.B, 64).tolist(), gen.integers(0, w.H, 64).tolist())))
    n_idx = torch.tensor([p[0] for p in pairs])
    h_idx = torch.tensor([p[1] for p in pairs])
    slots = torch.arange(steps) % ring

    def seq(x):   # [ring, N, H, d] -> [1, P, steps, d]
        return x[slots][:, n_idx, h_idx].permute(1, 0, 2).unsqueeze(0).contiguous()

    q, k, v = seq(inp["q"]), seq(inp["k"]), seq(inp["v"])
    beta = inp["beta"][slots][:, n_idx, h_idx].T.unsqueeze(0).contiguous()
    S0 = inp["S0"][n_idx, h_idx].unsqueeze(0)
    o_ref, S_ref = oracle.delta_recurrent(q, k, v, beta, None, S0=S0)
    assert_close(S[n_idx, h_idx], S_ref[0], TOL[w.dtype], "S after 1010 steps (sampled)")
    assert_close(o[n_idx, h_idx], o_ref[0, :, -1], TOL[w.dtype], "o of step 1010 (sampled)")


def test_token_gate_at_the_gated_workload_shape_full():
    """gated_deltanet_prefill (one decay per token) at B=1 H=32 T=32768
    d=128 bf16, the shape and launch its bench row times, on every head."""
    dev = require_gpu()
    w = W[3]
    print("gated_deltanet_prefill at the gated workload's shape", flush=True)
    inp = workloads.make_delta(w.B, w.H, w.T, w.dk, w.dv, w.dtype, seed=90 + w.index, gated="token")
    d = _to(inp, dev)
    o, S = la.gated_deltanet_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"])
    torch.cuda.synchronize()
    del d
    o_ref, S_ref = oracle.delta_recurrent(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"])
    assert_close(o, o_ref, TOL[w.dtype], "o (all heads)")
    assert_close(S, S_ref, TOL[w.dtype], "S (all heads)")


def test_gla_at_the_la_workload_shape():
    """gla_prefill at B=8 H=12 T=1024 d=64 bf16, the shape its bench row times."""
    dev = require_gpu()
    w = W[1]
    inp = workloads.make_gla(w.B, w.H, w.T, w.dk, w.dv, w.dtype, seed=92)
    d = _to(inp, dev)
    o, S = la.gla_prefill(d["q"], d["k"], d["v"], d["g"])
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.gla_recurrent(inp["q"], inp["k"], inp["v"], inp["g"])
    assert_close(o, o_ref, TOL[w.dtype], "o")
    assert_close(S, S_ref, TOL[w.dtype], "S")


def test_backward_at_the_deltanet_workload_shape_sampled_heads():
    """deltanet_prefill_backward at B=4 H=16 T=4096 d=128 bf16 (the shape its
    bench row times); the oracle's reverse recurrence on two sampled heads."""
    dev = require_gpu()
    w = W[2]
    print("deltanet_prefill_backward at the delta-rule workload's shape", flush=True)
    inp = workloads.make_delta(w.B, w.H, w.T, w.dk, w.dv, w.dtype, seed=95)
    gen = workloads.generator(96)
    dO = torch.randn(w.B, w.H, w.T, w.dv, generator=gen).to(w.dtype)
    d = _to(inp, dev)
    grads = la.deltanet_prefill_backward(d["q"], d["k"], d["v"], d["beta"], dO.to(dev))
    torch.cuda.synchronize()
    bi, heads = 1, [2, 13]
    sub = {n: inp[n][bi:bi + 1, heads].contiguous() for n in ("q", "k", "v", "beta")}
    ref = oracle.delta_backward(sub["q"], sub["k"], sub["v"], sub["beta"],
                                dO[bi:bi + 1, heads].contiguous())
    for name, g, r in zip(("dq", "dk", "dv", "dbeta"), grads, ref):
        assert_close(g[bi:bi + 1, heads], r, TOL[w.dtype], f"{name} (sampled heads)")


def test_gated_backward_at_the_deltanet_workload_shape_sampled_heads():
    """gated_deltanet_prefill_backward (one decay per token) at B=4 H=16
    T=4096 d=128 bf16, the shape and launch its bench row times (pass 1 is
    the pipelined per-token kernel with state capture over 64 chunks); the
    oracle's gated reverse recurrence on two sampled heads, dg included."""
    dev = require_gpu()
    w = W[2]
    print("gated_deltanet_prefill_backward at the delta-rule workload's shape", flush=True)
    inp = workloads.make_delta(w.B, w.H, w.T, w.dk, w.dv, w.dtype, seed=97, gated="token")
    gen = workloads.generator(98)
    dO = torch.randn(w.B, w.H, w.T, w.dv, generator=gen).to(w.dtype)
    d = _to(inp, dev)
    grads = la.gated_deltanet_prefill_backward(d["q"], d["k"], d["v"], d["beta"], d["g"], dO.to(dev))
    torch.cuda.synchronize()
    bi, heads = 2, [5, 14]
    sub = {n: inp[n][bi:bi + 1, heads].contiguous() for n in ("q", "k", "v", "beta", "g")}
    ref = oracle.delta_backward(sub["q"], sub["k"], sub["v"], sub["beta"],
                                dO[bi:bi + 1, heads].contiguous(), g=sub["g"])
    names = ("dq", "dk", "dv", "dbeta", "dg")
    ref = (ref[0], ref[1], ref[2], ref[3], ref[5])   # the oracle returns dS0 before dg
    for name, g, r in zip(names, grads[:5], ref):
        assert_close(g[bi:bi + 1, heads], r, TOL[w.dtype], f"{name} (sampled heads)")
