"""Caller-owned workspaces: the entry points that need scratch memory take a
torch-allocated device buffer of the size their *_workspace_bytes() query
returns.  Its contents on entry do not matter (it is filled with NaN bytes
here), a larger buffer works as well, and one buffer serves consecutive
calls on a stream; results equal the oracle's."""
import pytest
import torch

import delta_rule_recurrent_chunkwise_amd as la
import oracle
import workloads
from gpu_common import TOL, assert_close, require_gpu

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _garbage(nbytes, dev, extra=0):
    w = torch.empty(nbytes + extra, device=dev, dtype=torch.uint8)
    w.fill_(0xFF)   # every float read from it would be a NaN
    return w


def test_prefill_workspaces_reused_across_calls():
    dev = require_gpu()
    print("la_prefill, gla_prefill, gated deltanet_prefill with caller workspaces", flush=True)
    B, H, T, d = 2, 3, 200, 64
    la_in = workloads.make_la(B, H, T, d, d, BF, seed=301)
    gla_in = workloads.make_gla(B, H, T, d, d, BF, seed=302)
    kda_in = workloads.make_delta(1, 2, 150, 128, 128, BF, seed=303, gated=True)
    n = max(la.la_prefill_workspace_bytes(B, H, T, d, d, BF),
            la.gla_prefill_workspace_bytes(B, H, T, d, d, BF),
            la.deltanet_prefill_workspace_bytes(True, 1, 2, 150, 128, 128, BF))
    ws = _garbage(n, dev, extra=4096)
    for _ in range(2):
        x = {k: v.to(dev) for k, v in la_in.items()}
        o, S, z = la.la_prefill(x["q"], x["k"], x["v"], workspace=ws)
        x = {k: v.to(dev) for k, v in gla_in.items()}
        og, Sg = la.gla_prefill(x["q"], x["k"], x["v"], x["g"], workspace=ws)
        x = {k: v.to(dev) for k, v in kda_in.items()}
        ok, Sk = la.deltanet_prefill(x["q"], x["k"], x["v"], x["beta"], g=x["g"], workspace=ws)
        torch.cuda.synchronize()
        r = oracle.la_recurrent(la_in["q"], la_in["k"], la_in["v"])
        for name, g, ref in zip(("o", "S", "z"), (o, S, z), r):
            assert_close(g, ref, TOL[BF], f"la {name}")
        r = oracle.gla_recurrent(gla_in["q"], gla_in["k"], gla_in["v"], gla_in["g"])
        assert_close(og, r[0], TOL[BF], "gla o")
        assert_close(Sg, r[1], TOL[BF], "gla S")
        r = oracle.delta_recurrent(kda_in["q"], kda_in["k"], kda_in["v"], kda_in["beta"], kda_in["g"])
        assert_close(ok, r[0], TOL[BF], "gated o")
        assert_close(Sk, r[1], TOL[BF], "gated S")
        ws.fill_(0xFF)


def test_backward_workspace_given_by_the_caller():
    dev = require_gpu()
    print("deltanet_prefill_backward with a caller workspace", flush=True)
    B, H, T, d = 1, 2, 130, 128
    inp = workloads.make_delta(B, H, T, d, d, BF, seed=304)
    dO = torch.randn(B, H, T, d, generator=workloads.generator(305)).to(BF)
    n = la.deltanet_prefill_backward_workspace_bytes(B, H, T, d, d, BF)
    ws = _garbage(n, dev)
    x = {k: v.to(dev) for k, v in inp.items()}
    grads = la.deltanet_prefill_backward(x["q"], x["k"], x["v"], x["beta"], dO.to(dev), workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.delta_backward(inp["q"], inp["k"], inp["v"], inp["beta"], dO)
    for name, g, r in zip(("dq", "dk", "dv", "dbeta"), grads, ref):
        assert_close(g, r, TOL[BF], name)


def test_too_small_workspace_raises_before_launch():
    dev = require_gpu()
    B, H, T, d = 1, 2, 64, 64
    q = torch.zeros(B, H, T, d, device=dev, dtype=BF)
    n = la.la_prefill_workspace_bytes(B, H, T, d, d, BF)
    with pytest.raises(la.LinAttnError) as e:
        la.la_prefill(q, q, q, workspace=torch.empty(n - 1, device=dev, dtype=torch.uint8))
    assert e.value.code == -7
