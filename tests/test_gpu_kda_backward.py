"""kda_prefill_backward (a decay per key channel) on the GPU against the
float64 oracle's gated reverse-mode recurrence (pinned to finite differences
and torch autograd), through the C ABI: every dimension pair, with and
without an initial state and a final-state gradient, ragged lengths, the
chain's prefetch loop, chunks whose decay leaves the factored form's range
(every chunk, one channel of one chunk, growth), the per-token rule as the
special case of equal channels, no decay as the ungated rule, and the gated
workload's shape on sampled heads."""
import pytest
import torch

import delta_rule_recurrent_chunkwise_amd as la
import oracle
import workloads
from gpu_common import TOL, assert_close, require_gpu

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
DIMS = [(16, 16), (32, 64), (64, 32), (64, 64), (128, 128), (128, 16), (16, 128), (128, 64)]
NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dS0")


def _run(inp, dO, dST, init, what):
    dev = require_gpu()
    d = {n: t.to(dev) for n, t in inp.items()}
    grads = la.kda_prefill_backward(d["q"], d["k"], d["v"], d["beta"], d["g"], dO.to(dev),
                                    S0=d["S0"] if init else None,
                                    dST=dST.to(dev) if dST is not None else None, want_dS0=True)
    torch.cuda.synchronize()
    dq, dk_, dv_, db, dS0, dg = oracle.delta_backward(
        inp["q"], inp["k"], inp["v"], inp["beta"], dO, S0=inp["S0"] if init else None, dST=dST,
        g=inp["g"])
    for name, g, r in zip(NAMES, grads, (dq, dk_, dv_, db, dg, dS0)):
        assert_close(g, r, TOL[BF16], f"{name} {what}")
    return grads


def _inputs(B, H, T, dk, dv, seed, init, with_dst, gscale=1.0):
    inp = workloads.make_delta(B, H, T, dk, dv, BF16, seed=seed, gated=True, init_state=init,
                               state_std=0.5)
    if gscale != 1.0:
        inp["g"] = (inp["g"].float() * gscale).to(BF16)
    gen = workloads.generator(seed + 1)
    dO = torch.randn(B, H, T, dv, generator=gen).to(BF16)
    dST = 0.5 * torch.randn(B, H, dk, dv, generator=gen) if with_dst else None
    return inp, dO, dST


def _check(B, H, T, dk, dv, seed, init, with_dst, gscale=1.0):
    print(f"  kda backward B={B} H={H} T={T} dk={dk} dv={dv} init={init} dST={with_dst} "
          f"gscale={gscale}", flush=True)
    inp, dO, dST = _inputs(B, H, T, dk, dv, seed, init, with_dst, gscale)
    return _run(inp, dO, dST, init, f"T={T}")


@pytest.mark.parametrize("dk,dv", DIMS)
@pytest.mark.parametrize("init", [False, True], ids=["zero", "init"])
def test_kda_backward(dk, dv, init):
    _check(2, 3, 192, dk, dv, 1400 + dk + 3 * dv, init, init, gscale=8.0)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 32)])
def test_kda_backward_ragged(dk, dv):
    for B, H, T in ((2, 3, 1), (2, 3, 63), (2, 3, 100), (4, 16, 130)):
        _check(B, H, T, dk, dv, 1500 + T, True, True)


@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 32), (128, 16), (128, 128)])
def test_kda_backward_chain_loop(dk, dv):
    """Six chunks and a ragged tail: every slot of the chain's prefetch ring
    carries its own per-channel chunk decay."""
    _check(1, 2, 327, dk, dv, 1600 + dk + dv, True, True, gscale=4.0)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 32), (16, 16), (128, 16)])
@pytest.mark.parametrize("gval", [-3.0, -40.0])
def test_kda_backward_strong_decay_every_chunk(dk, dv, gval):
    """-3 per token and channel sums to -192 over a chunk, -40 all but clears
    the state at every token: every chunk is out of the factored form's range
    and is computed from the recurrence."""
    print(f"  kda backward g={gval} dk={dk} dv={dv}", flush=True)
    inp, dO, dST = _inputs(1, 2, 150, dk, dv, 1700 + dk, True, True)
    inp["g"] = torch.full_like(inp["g"], gval)
    _run(inp, dO, dST, True, f"g={gval}")


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (32, 16)])
def test_kda_backward_burst_in_one_channel_of_one_chunk(dk, dv):
    """Mild decays except channel 5 of tokens 70 .. 99 at -9 per token: chunk
    1 is computed from the recurrence, chunks 0 and 2 in the factored form,
    and the gradient crosses between them."""
    inp, dO, dST = _inputs(1, 3, 200, dk, dv, 1800 + dk + dv, True, True)
    g = inp["g"].clone()
    g[:, :, 70:100, 5] = -9.0
    inp["g"] = g
    _run(inp, dO, dST, True, "burst")


def test_kda_backward_growth():
    """g > 0 (growth) in channel 3 of chunk 2, 1.1 per token: out of range,
    from the recurrence, next to factored chunks."""
    inp, dO, dST = _inputs(1, 2, 256, 128, 64, 1900, True, True)
    g = inp["g"].clone()
    g[:, :, 128:192, 3] = 1.1
    inp["g"] = g
    _run(inp, dO, dST, True, "growth")


def test_kda_backward_equal_channels_is_the_per_token_rule():
    """A per-channel decay equal in every channel is the per-token rule:
    dq, dk, dv, dbeta and dS0 of gated_deltanet_prefill_backward, and dg
    summed over the channels equal to its dg."""
    dev = require_gpu()
    tok = workloads.make_delta(2, 3, 150, 128, 64, BF16, seed=2000, gated="token",
                               init_state=True, state_std=0.5)
    g_tok = (tok["g"].float() * 4.0).to(BF16)
    g_ch = g_tok[..., None].expand(2, 3, 150, 128).contiguous()
    gen = workloads.generator(2001)
    dO = torch.randn(2, 3, 150, 64, generator=gen).to(BF16)
    d = {n: t.to(dev) for n, t in tok.items()}
    a = la.kda_prefill_backward(d["q"], d["k"], d["v"], d["beta"], g_ch.to(dev), dO.to(dev),
                                S0=d["S0"], want_dS0=True)
    b = la.gated_deltanet_prefill_backward(d["q"], d["k"], d["v"], d["beta"], g_tok.to(dev),
                                           dO.to(dev), S0=d["S0"], want_dS0=True)
    torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk", "dv", "dbeta"), a[:4], b[:4]):
        assert_close(x, y, TOL[BF16], f"{name} equal channels")
    assert_close(a[5], b[5], TOL[BF16], "dS0 equal channels")
    assert_close(a[4].float().sum(-1), b[4], TOL[BF16], "dg summed over channels")


def test_kda_backward_zero_gate_is_ungated():
    dev = require_gpu()
    inp, dO, _ = _inputs(2, 3, 150, 128, 64, 2100, True, False)
    inp["g"] = torch.zeros_like(inp["g"])
    d = {n: t.to(dev) for n, t in inp.items()}
    a = la.kda_prefill_backward(d["q"], d["k"], d["v"], d["beta"], d["g"], dO.to(dev),
                                S0=d["S0"], want_dS0=True)
    b = la.deltanet_prefill_backward(d["q"], d["k"], d["v"], d["beta"], dO.to(dev), S0=d["S0"],
                                     want_dS0=True)
    torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk", "dv", "dbeta", "dS0"), a[:4] + a[5:], b):
        assert_close(x, y, TOL[BF16], f"{name} g=0")
    ref = oracle.delta_backward(inp["q"], inp["k"], inp["v"], inp["beta"], dO, S0=inp["S0"],
                                g=inp["g"])
    assert_close(a[4], ref[5], TOL[BF16], "dg g=0")


def test_kda_backward_of_empty_sequence():
    dev = require_gpu()
    e = torch.empty(1, 2, 0, 32, device=dev, dtype=BF16)
    eb = torch.empty(1, 2, 0, device=dev, dtype=BF16)
    dST = torch.randn(1, 2, 32, 32, device=dev)
    out = la.kda_prefill_backward(e, e, e, eb, e, e, dST=dST, want_dS0=True)
    torch.cuda.synchronize()
    assert torch.equal(out[5], dST)
    assert out[4].numel() == 0


def test_kda_backward_rejects_float32():
    dev = require_gpu()
    x = torch.zeros(1, 1, 64, 16, device=dev)
    b = torch.zeros(1, 1, 64, device=dev)
    with pytest.raises(la.LinAttnError):
        la.kda_prefill_backward(x, x, x, b, x, x)


def test_kda_backward_at_the_gated_workload_shape_sampled_heads():
    """B=1 H=32 T=32768 d=128 with the gated workload's decays: the GPU runs
    all 32 heads (pipelined forward with state capture, 512 chunks per head
    in the chain); the oracle checks four of them (heads are independent)."""
    dev = require_gpu()
    w = workloads.WORKLOADS[3]
    inp = workloads.make_workload(w)
    gen = workloads.generator(2200)
    dO = torch.randn(w.B, w.H, w.T, w.dv, generator=gen).to(BF16)
    d = {n: t.to(dev) for n, t in inp.items()}
    grads = la.kda_prefill_backward(d["q"], d["k"], d["v"], d["beta"], d["g"], dO.to(dev),
                                    want_dS0=True)
    torch.cuda.synchronize()
    heads = [0, 9, 21, 31]
    sub = {n: t[:, heads].contiguous() for n, t in inp.items() if n != "S0"}
    ref = oracle.delta_backward(sub["q"], sub["k"], sub["v"], sub["beta"],
                                dO[:, heads].contiguous(), g=sub["g"])
    ref = (ref[0], ref[1], ref[2], ref[3], ref[5], ref[4])
    for name, g, r in zip(NAMES, grads, ref):
        assert_close(g[:, heads], r, TOL[BF16], f"{name} (sampled heads)")
