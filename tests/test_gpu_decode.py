"""Decode steps on the GPU against the float64 oracle (one-token recurrence
steps chained through the state), through the C ABI."""
import numpy as np
import pytest
import torch

import delta_rule_recurrent_chunkwise_amd as la
import oracle
import workloads
from gpu_common import TOL, assert_close, require_gpu

pytestmark = pytest.mark.gpu

DIMS = [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16), (16, 128), (64, 64)]
DTYPES = [torch.float32, torch.bfloat16]


def _slot(x, s):
    return x[s].contiguous()


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", DIMS)
@pytest.mark.parametrize("gated", [False, True], ids=["delta", "gated"])
def test_deltanet_decode_steps(dtype, dk, dv, gated):
    dev = require_gpu()
    N, H, steps = 5, 3, 3
    inp = workloads.make_decode(N, H, dk, dv, dtype, seed=11 + dk + dv, gated=gated,
                                ring=steps)
    S = inp["S0"].to(dev)
    S_ref = inp["S0"].double().numpy()
    for s in range(steps):
        q, k, v, beta = (_slot(inp[n], s) for n in ("q", "k", "v", "beta"))
        g = _slot(inp["g"], s) if gated else None
        o = la.deltanet_decode_step(q.to(dev), k.to(dev), v.to(dev), beta.to(dev), S,
                                    g=g.to(dev) if gated else None)
        o_ref, S_ref = oracle.delta_recurrent(
            q[:, :, None], k[:, :, None], v[:, :, None], beta[:, :, None],
            g[:, :, None] if gated else None, S0=S_ref)
        torch.cuda.synchronize()
        assert_close(o, o_ref[:, :, 0], TOL[dtype], f"o step {s}")
        assert_close(S, S_ref, TOL[dtype] / 10, f"S step {s}")


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", DIMS)
def test_la_decode_steps(dtype, dk, dv):
    dev = require_gpu()
    N, H, steps = 5, 3, 3
    inp = workloads.make_la_decode(N, H, dk, dv, dtype, seed=23 + dk + dv, ring=steps)
    S, z = inp["S0"].to(dev), inp["z0"].to(dev)
    S_ref, z_ref = inp["S0"].double().numpy(), inp["z0"].double().numpy()
    for s in range(steps):
        q, k, v = (_slot(inp[n], s) for n in ("q", "k", "v"))
        o = la.la_decode_step(q.to(dev), k.to(dev), v.to(dev), S, z)
        o_ref, S_ref, z_ref = oracle.la_recurrent(q[:, :, None], k[:, :, None],
                                                  v[:, :, None], S_ref, z_ref)
        torch.cuda.synchronize()
        assert_close(o, o_ref[:, :, 0], TOL[dtype], f"o step {s}")
        assert_close(S, S_ref, TOL[dtype] / 10, f"S step {s}")
        assert_close(z, z_ref, TOL[dtype] / 10, f"z step {s}")


def test_decode_beta_zero_leaves_state_unchanged():
    dev = require_gpu()
    inp = workloads.make_decode(4, 2, 128, 128, torch.bfloat16, seed=5, ring=1)
    S = inp["S0"].to(dev)
    S0 = S.clone()
    beta = torch.zeros_like(inp["beta"][0])
    o = la.deltanet_decode_step(inp["q"][0].to(dev), inp["k"][0].to(dev),
                                inp["v"][0].to(dev), beta.to(dev), S)
    torch.cuda.synchronize()
    assert torch.equal(S, S0)
    ref = torch.einsum("nhd,nhde->nhe", inp["q"][0].double(), S0.cpu().double())
    assert_close(o, ref, TOL[torch.bfloat16], "o = q S0")


def test_decode_handles_many_heads_and_partial_blocks():
    """Head counts that leave the last workgroup partly empty."""
    dev = require_gpu()
    for dk, dv, N, H in [(16, 16, 7, 9), (64, 64, 3, 5), (32, 16, 1, 1)]:
        inp = workloads.make_decode(N, H, dk, dv, torch.float32, seed=N * H, ring=1)
        S = inp["S0"].to(dev)
        o = la.deltanet_decode_step(inp["q"][0].to(dev), inp["k"][0].to(dev),
                                    inp["v"][0].to(dev), inp["beta"][0].to(dev), S)
        o_ref, S_ref = oracle.delta_recurrent(
            inp["q"][0][:, :, None], inp["k"][0][:, :, None], inp["v"][0][:, :, None],
            inp["beta"][0][:, :, None], None, S0=inp["S0"])
        torch.cuda.synchronize()
        assert_close(o, o_ref[:, :, 0], 1e-4, f"o N={N} H={H} dk={dk}")
        assert_close(S, S_ref, 1e-5, f"S N={N} H={H} dk={dk}")
