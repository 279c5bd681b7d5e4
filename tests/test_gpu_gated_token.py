"""The per-token gated entry points on the GPU against the float64 oracle,
through the C ABI: gated_deltanet_prefill / gated_deltanet_decode_step (the
delta rule with one decay per token, Gated DeltaNet) and gla_prefill /
gla_decode_step (the additive cache with a forgetting factor), at sizes that
span several 64-token chunks, with ragged lengths and decays far beyond the
range of the per-channel chunk form."""
import pytest
import torch

import delta_rule_recurrent_chunkwise_amd as la
import oracle
import workloads
from gpu_common import TOL, assert_close, require_gpu

pytestmark = pytest.mark.gpu

DIMS = [(16, 16), (32, 64), (64, 32), (64, 64), (128, 128), (128, 16), (16, 128)]
DTYPES = [torch.float32, torch.bfloat16]
IDS = ["f32", "bf16"]


def _dev(d, dev):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def _gdn(inp, dev, init):
    d = _dev(inp, dev)
    o, S = la.gated_deltanet_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"],
                                     S=d["S0"].clone() if init else None,
                                     use_initial_state=init)
    torch.cuda.synchronize()
    ref = oracle.delta_recurrent(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"],
                                 S0=inp["S0"] if init else None)
    return (o, S), ref


def _gla(inp, dev, init, with_g=True):
    d = _dev(inp, dev)
    g = d["g"] if with_g else None
    o, S = la.gla_prefill(d["q"], d["k"], d["v"], g, S=d["S0"].clone() if init else None,
                          use_initial_state=init)
    torch.cuda.synchronize()
    ref = oracle.gla_recurrent(inp["q"], inp["k"], inp["v"], inp["g"] if with_g else None,
                               S0=inp["S0"] if init else None)
    return (o, S), ref


@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
@pytest.mark.parametrize("dk,dv", DIMS)
@pytest.mark.parametrize("init", [False, True], ids=["zero", "init"])
def test_gated_deltanet_prefill(dtype, dk, dv, init):
    dev = require_gpu()
    inp = workloads.make_delta(2, 3, 192, dk, dv, dtype, seed=300 + dk + 3 * dv,
                               gated="token", init_state=init, state_std=0.5)
    (o, S), (o_ref, S_ref) = _gdn(inp, dev, init)
    assert_close(o, o_ref, TOL[dtype], "o")
    assert_close(S, S_ref, TOL[dtype], "S")


@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
@pytest.mark.parametrize("dk,dv", DIMS)
@pytest.mark.parametrize("init", [False, True], ids=["zero", "init"])
def test_gla_prefill(dtype, dk, dv, init):
    dev = require_gpu()
    inp = workloads.make_gla(2, 3, 192, dk, dv, dtype, seed=400 + dk + 3 * dv,
                             init_state=init)
    (o, S), (o_ref, S_ref) = _gla(inp, dev, init)
    assert_close(o, o_ref, TOL[dtype], "o")
    assert_close(S, S_ref, TOL[dtype], "S")


@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
def test_gla_without_decay(dtype):
    """g = NULL: plain additive linear attention without a normaliser."""
    dev = require_gpu()
    inp = workloads.make_gla(1, 2, 130, 64, 64, dtype, seed=41, init_state=True)
    (o, S), (o_ref, S_ref) = _gla(inp, dev, True, with_g=False)
    assert_close(o, o_ref, TOL[dtype], "o")
    assert_close(S, S_ref, TOL[dtype], "S")


@pytest.mark.parametrize("dtype,dk,dv", [(torch.bfloat16, 128, 128), (torch.bfloat16, 64, 32),
                                         (torch.float32, 128, 64)],
                         ids=["bf16-128x128", "bf16-64x32", "f32-128x64"])
def test_many_heads_and_ragged(dtype, dk, dv):
    """Enough heads for the wide value slices, and T not a multiple of 64."""
    dev = require_gpu()
    for B, H, T in ((8, 32, 128), (2, 3, 1), (2, 3, 63), (2, 3, 100)):
        print(f"  B={B} H={H} T={T}", flush=True)
        inp = workloads.make_delta(B, H, T, dk, dv, dtype, seed=T + dk, gated="token",
                                   init_state=True, state_std=0.5)
        (o, S), (o_ref, S_ref) = _gdn(inp, dev, True)
        assert_close(o, o_ref, TOL[dtype], f"gdn o T={T}")
        assert_close(S, S_ref, TOL[dtype], f"gdn S T={T}")
        inp = workloads.make_gla(B, H, T, dk, dv, dtype, seed=T + dk + 1, init_state=True)
        (o, S), (o_ref, S_ref) = _gla(inp, dev, True)
        assert_close(o, o_ref, TOL[dtype], f"gla o T={T}")
        assert_close(S, S_ref, TOL[dtype], f"gla S T={T}")


@pytest.mark.parametrize("dtype,dk,dv", [(torch.bfloat16, 128, 128), (torch.float32, 64, 64)],
                         ids=["bf16-128", "f32-64"])
@pytest.mark.parametrize("gval", [-3.0, -40.0])
def test_strong_decay(dtype, dk, dv, gval):
    """A uniform log-decay of -3 per token sums to -192 over a chunk (the
    per-channel chunk form overflows beyond about -87); -40 per token all
    but clears the state at every step.  Both still match the oracle."""
    dev = require_gpu()
    inp = workloads.make_delta(1, 2, 160, dk, dv, dtype, seed=7, gated="token",
                               init_state=True, state_std=0.5)
    inp["g"] = torch.full_like(inp["g"], gval)
    (o, S), (o_ref, S_ref) = _gdn(inp, dev, True)
    assert_close(o, o_ref, TOL[dtype], "gdn o")
    assert_close(S, S_ref, TOL[dtype], "gdn S")
    inp = workloads.make_gla(1, 2, 160, dk, dv, dtype, seed=8, init_state=True)
    inp["g"] = torch.full_like(inp["g"], gval)
    (o, S), (o_ref, S_ref) = _gla(inp, dev, True)
    assert_close(o, o_ref, TOL[dtype], "gla o")
    assert_close(S, S_ref, TOL[dtype], "gla S")


def test_token_gate_equals_channel_broadcast():
    """gated_deltanet_prefill equals deltanet_prefill with the same decay for
    every key channel (two different chunk algorithms)."""
    dev = require_gpu()
    inp = workloads.make_delta(2, 4, 256, 128, 128, torch.bfloat16, seed=12, gated="token",
                               init_state=True, state_std=0.5)
    d = _dev(inp, dev)
    o1, S1 = la.gated_deltanet_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"],
                                       S=d["S0"].clone(), use_initial_state=True)
    gch = d["g"][..., None].expand(-1, -1, -1, 128).contiguous()
    o2, S2 = la.deltanet_prefill(d["q"], d["k"], d["v"], d["beta"], g=gch, S=d["S0"].clone(),
                                 use_initial_state=True)
    torch.cuda.synchronize()
    assert_close(o1, o2.float(), 2e-2, "o")
    assert_close(S1, S2, 2e-2, "S")


@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
@pytest.mark.parametrize("dk,dv", [(64, 32), (128, 128)])
def test_decode_steps(dtype, dk, dv):
    """Five one-token decode calls equal the oracle over the five tokens, for
    both per-token gated rules (and gated linear attention without a decay)."""
    dev = require_gpu()
    N, H, T = 3, 4, 5
    inp = workloads.make_delta(N, H, T, dk, dv, dtype, seed=dk + dv, gated="token",
                               init_state=True, state_std=0.5)
    S = inp["S0"].to(dev)
    outs = []
    for t in range(T):
        x = {n: inp[n][:, :, t].contiguous().to(dev) for n in ("q", "k", "v", "beta", "g")}
        outs.append(la.gated_deltanet_decode_step(x["q"], x["k"], x["v"], x["beta"], x["g"], S))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.delta_recurrent(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"],
                                          S0=inp["S0"])
    assert_close(torch.stack(outs, 2), o_ref, TOL[dtype], "gdn decode o")
    assert_close(S, S_ref, TOL[dtype], "gdn decode S")
    for with_g in (True, False):
        gi = workloads.make_gla(N, H, T, dk, dv, dtype, seed=dk + dv + 1, init_state=True)
        S = gi["S0"].to(dev)
        outs = []
        for t in range(T):
            x = {n: gi[n][:, :, t].contiguous().to(dev) for n in ("q", "k", "v", "g")}
            outs.append(la.gla_decode_step(x["q"], x["k"], x["v"], S,
                                           g=x["g"] if with_g else None))
        torch.cuda.synchronize()
        o_ref, S_ref = oracle.gla_recurrent(gi["q"], gi["k"], gi["v"],
                                            gi["g"] if with_g else None, S0=gi["S0"])
        assert_close(torch.stack(outs, 2), o_ref, TOL[dtype], f"gla decode o g={with_g}")
        assert_close(S, S_ref, TOL[dtype], f"gla decode S g={with_g}")


@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
def test_split_prefill_equals_full(dtype):
    """Two prefills chained through the returned state equal one over the
    concatenated tokens, for both entry points."""
    dev = require_gpu()
    inp = workloads.make_delta(1, 3, 320, 128, 64, dtype, seed=55, gated="token")
    d = _dev(inp, dev)
    o, S = la.gated_deltanet_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"])
    cut = 192
    part = lambda x, a, b: x[:, :, a:b].contiguous()  # noqa: E731
    o1, S1 = la.gated_deltanet_prefill(*(part(d[n], 0, cut) for n in ("q", "k", "v", "beta", "g")))
    o2, S2 = la.gated_deltanet_prefill(*(part(d[n], cut, 320) for n in ("q", "k", "v", "beta", "g")),
                                       S=S1, use_initial_state=True)
    torch.cuda.synchronize()
    assert_close(torch.cat([o1, o2], 2), o.float(), 1e-5, "gdn o")
    assert_close(S2, S, 1e-5, "gdn S")
    gi = _dev(workloads.make_gla(1, 3, 320, 128, 64, dtype, seed=56), dev)
    o, S = la.gla_prefill(gi["q"], gi["k"], gi["v"], gi["g"])
    o1, S1 = la.gla_prefill(*(part(gi[n], 0, cut) for n in ("q", "k", "v", "g")))
    o2, S2 = la.gla_prefill(*(part(gi[n], cut, 320) for n in ("q", "k", "v", "g")), S=S1,
                            use_initial_state=True)
    torch.cuda.synchronize()
    assert_close(torch.cat([o1, o2], 2), o.float(), 1e-5, "gla o")
    assert_close(S2, S, 1e-5, "gla S")
