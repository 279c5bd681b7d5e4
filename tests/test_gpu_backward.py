"""deltanet_prefill_backward on the GPU against the float64 oracle's
reverse-mode recurrence (itself pinned to finite differences and to torch
autograd), through the C ABI: every dimension pair, both dtypes, with and
without an initial state and a final-state gradient, ragged lengths."""
import pytest
import torch

import delta_rule_recurrent_chunkwise_amd as la
import oracle
import workloads
from gpu_common import TOL, assert_close, require_gpu

pytestmark = pytest.mark.gpu

DIMS_BF16 = [(16, 16), (32, 64), (64, 32), (64, 64), (128, 128), (128, 16), (16, 128)]
DIMS_F32 = [(16, 16), (32, 64), (64, 32), (64, 64)]


def _check(B, H, T, dk, dv, dtype, seed, init, with_dst):
    dev = require_gpu()
    inp = workloads.make_delta(B, H, T, dk, dv, dtype, seed=seed, init_state=init, state_std=0.5)
    gen = workloads.generator(seed + 1)
    dO = torch.randn(B, H, T, dv, generator=gen).to(dtype)
    dST = 0.5 * torch.randn(B, H, dk, dv, generator=gen) if with_dst else None
    d = {n: t.to(dev) for n, t in inp.items()}
    grads = la.deltanet_prefill_backward(d["q"], d["k"], d["v"], d["beta"], dO.to(dev),
                                         S0=d["S0"] if init else None,
                                         dST=dST.to(dev) if with_dst else None, want_dS0=True)
    torch.cuda.synchronize()
    ref = oracle.delta_backward(inp["q"], inp["k"], inp["v"], inp["beta"], dO,
                                S0=inp["S0"] if init else None, dST=dST)
    for name, g, r in zip(("dq", "dk", "dv", "dbeta", "dS0"), grads, ref):
        assert_close(g, r, TOL[dtype], f"{name} T={T}")


@pytest.mark.parametrize("dk,dv", DIMS_BF16)
@pytest.mark.parametrize("init", [False, True], ids=["zero", "init"])
def test_backward_bf16(dk, dv, init):
    _check(2, 3, 192, dk, dv, torch.bfloat16, 500 + dk + 3 * dv, init, init)


@pytest.mark.parametrize("dk,dv", DIMS_F32)
@pytest.mark.parametrize("init", [False, True], ids=["zero", "init"])
def test_backward_f32(dk, dv, init):
    _check(2, 3, 192, dk, dv, torch.float32, 600 + dk + 3 * dv, init, not init)


@pytest.mark.parametrize("dtype,dk,dv", [(torch.bfloat16, 128, 128), (torch.float32, 64, 64)],
                         ids=["bf16-128", "f32-64"])
def test_backward_ragged_and_many_heads(dtype, dk, dv):
    for B, H, T in ((2, 3, 1), (2, 3, 63), (2, 3, 100), (4, 16, 128)):
        print(f"  B={B} H={H} T={T}", flush=True)
        _check(B, H, T, dk, dv, dtype, 700 + T, True, True)


@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 32), (16, 128), (128, 16), (128, 128)])
def test_backward_long_enough_for_the_chain_loop(dk, dv):
    """Six chunks and a ragged tail (T = 327): the reverse chain's prefetch
    ring runs its main loop (four chunks) and its tail, at every width of
    the value slices (16 and 32 columns) and the 16-deep product (dk = 16)."""
    _check(1, 2, 327, dk, dv, torch.bfloat16, 800 + dk + dv, True, True)


def test_backward_of_empty_sequence():
    """T = 0: the initial state's gradient is the final state's."""
    dev = require_gpu()
    e = torch.empty(1, 2, 0, 32, device=dev, dtype=torch.bfloat16)
    eb = torch.empty(1, 2, 0, device=dev, dtype=torch.bfloat16)
    dST = torch.randn(1, 2, 32, 32, device=dev)
    _, _, _, _, dS0 = la.deltanet_prefill_backward(e, e, e, eb, e, dST=dST, want_dS0=True)
    torch.cuda.synchronize()
    assert torch.equal(dS0, dST)
    _, _, _, _, dS0 = la.deltanet_prefill_backward(e, e, e, eb, e, want_dS0=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dS0) == 0
