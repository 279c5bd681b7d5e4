"""gated_deltanet_prefill_backward (one decay per token) on the GPU against
the float64 oracle's gated reverse-mode recurrence (pinned to finite
differences, torch autograd and the rescaling identity for dg), through the
C ABI: every dimension pair, both dtypes, with and without an initial state
and a final-state gradient, ragged lengths, the chain's prefetch loop, and
decays far beyond what a chunk-level rescaling could hold."""
import pytest
import torch

import delta_rule_recurrent_chunkwise_amd as la
import oracle
import workloads
from gpu_common import TOL, assert_close, require_gpu

pytestmark = pytest.mark.gpu

DIMS_BF16 = [(16, 16), (32, 64), (64, 32), (64, 64), (128, 128), (128, 16), (16, 128)]
DIMS_F32 = [(16, 16), (32, 64), (64, 32), (64, 64)]
NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dS0")


def _check(B, H, T, dk, dv, dtype, seed, init, with_dst, gval=None, gscale=1.0):
    dev = require_gpu()
    inp = workloads.make_delta(B, H, T, dk, dv, dtype, seed=seed, gated="token",
                               init_state=init, state_std=0.5)
    if gval is not None:
        inp["g"] = torch.full_like(inp["g"], gval)
    elif gscale != 1.0:
        inp["g"] = (inp["g"].float() * gscale).to(dtype)
    gen = workloads.generator(seed + 1)
    dO = torch.randn(B, H, T, dv, generator=gen).to(dtype)
    dST = 0.5 * torch.randn(B, H, dk, dv, generator=gen) if with_dst else None
    d = {n: t.to(dev) for n, t in inp.items()}
    print(f"  B={B} H={H} T={T} dk={dk} dv={dv} {dtype} init={init} dST={with_dst} g={gval}",
          flush=True)
    grads = la.gated_deltanet_prefill_backward(d["q"], d["k"], d["v"], d["beta"], d["g"],
                                               dO.to(dev), S0=d["S0"] if init else None,
                                               dST=dST.to(dev) if with_dst else None,
                                               want_dS0=True)
    torch.cuda.synchronize()
    dq, dk_, dv_, db, dS0, dg = oracle.delta_backward(
        inp["q"], inp["k"], inp["v"], inp["beta"], dO, S0=inp["S0"] if init else None,
        dST=dST, g=inp["g"])
    for name, g, r in zip(NAMES, grads, (dq, dk_, dv_, db, dg, dS0)):
        assert_close(g, r, TOL[dtype], f"{name} T={T}")


@pytest.mark.parametrize("dk,dv", DIMS_BF16)
@pytest.mark.parametrize("init", [False, True], ids=["zero", "init"])
def test_gated_backward_bf16(dk, dv, init):
    _check(2, 3, 192, dk, dv, torch.bfloat16, 900 + dk + 3 * dv, init, init, gscale=8.0)


@pytest.mark.parametrize("dk,dv", DIMS_F32)
@pytest.mark.parametrize("init", [False, True], ids=["zero", "init"])
def test_gated_backward_f32(dk, dv, init):
    _check(2, 3, 192, dk, dv, torch.float32, 950 + dk + 3 * dv, init, not init, gscale=8.0)


@pytest.mark.parametrize("dtype,dk,dv", [(torch.bfloat16, 128, 128), (torch.float32, 64, 64)],
                         ids=["bf16-128", "f32-64"])
def test_gated_backward_ragged(dtype, dk, dv):
    for B, H, T in ((2, 3, 1), (2, 3, 63), (2, 3, 100), (4, 16, 130)):
        _check(B, H, T, dk, dv, dtype, 1000 + T, True, True)


@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 32), (128, 16), (128, 128)])
def test_gated_backward_chain_loop(dk, dv):
    """Six chunks and a ragged tail: every slot of the chain's prefetch ring
    carries its own chunk decay."""
    _check(1, 2, 327, dk, dv, torch.bfloat16, 1100 + dk + dv, True, True, gscale=4.0)


@pytest.mark.parametrize("dtype,dk,dv", [(torch.bfloat16, 128, 128), (torch.float32, 64, 64)],
                         ids=["bf16-128", "f32-64"])
@pytest.mark.parametrize("gval", [-3.0, -40.0])
def test_gated_backward_strong_decay(dtype, dk, dv, gval):
    """-3 per token sums to -192 over a chunk, -40 all but clears the state at
    every token: only decay ratios of at most 1 are ever formed."""
    _check(1, 2, 160, dk, dv, dtype, 1200, True, True, gval=gval)


def test_gated_backward_zero_gate_is_ungated():
    """g = 0: the gradients of the ungated entry point, and dg equal to the
    rescaling identity's sums (checked against the oracle)."""
    dev = require_gpu()
    inp = workloads.make_delta(2, 3, 150, 128, 64, torch.bfloat16, seed=1300, gated="token",
                               init_state=True, state_std=0.5)
    inp["g"] = torch.zeros_like(inp["g"])
    gen = workloads.generator(1301)
    dO = torch.randn(2, 3, 150, 64, generator=gen).to(torch.bfloat16)
    d = {n: t.to(dev) for n, t in inp.items()}
    gated = la.gated_deltanet_prefill_backward(d["q"], d["k"], d["v"], d["beta"], d["g"],
                                               dO.to(dev), S0=d["S0"], want_dS0=True)
    plain = la.deltanet_prefill_backward(d["q"], d["k"], d["v"], d["beta"], dO.to(dev),
                                         S0=d["S0"], want_dS0=True)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "dbeta", "dS0"), gated[:4] + gated[5:], plain):
        assert_close(a, b, TOL[torch.bfloat16], f"{name} g=0")
    ref = oracle.delta_backward(inp["q"], inp["k"], inp["v"], inp["beta"], dO, S0=inp["S0"],
                                g=inp["g"])
    assert_close(gated[4], ref[5], TOL[torch.bfloat16], "dg g=0")


def test_gated_backward_of_empty_sequence():
    dev = require_gpu()
    e = torch.empty(1, 2, 0, 32, device=dev, dtype=torch.bfloat16)
    eb = torch.empty(1, 2, 0, device=dev, dtype=torch.bfloat16)
    dST = torch.randn(1, 2, 32, 32, device=dev)
    out = la.gated_deltanet_prefill_backward(e, e, e, eb, eb, e, dST=dST, want_dS0=True)
    torch.cuda.synchronize()
    assert torch.equal(out[5], dST)
    assert out[4].numel() == 0
