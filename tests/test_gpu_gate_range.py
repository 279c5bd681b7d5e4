"""The per-key-channel gated delta rule (deltanet_prefill with g) where the
decay inside a 64-token chunk is too strong for the factored chunk form
(K / Gam would leave the float range): such chunks are computed token by
token, so the result still equals the oracle's recurrence.  Covered on the
pipelined kernel (bf16, dk = 128) and the generic kernel (float32 and bf16,
dk <= 64, and dv = 16), for a decay of -3 and -40 per token and channel (every
chunk out of range), for a mild workload with one burst of strong decay in a
single channel of one chunk (the other chunks in range), and for growth
(g > 0)."""
import pytest
import torch

import delta_rule_recurrent_chunkwise_amd as la
import oracle
import workloads
from gpu_common import TOL, assert_close, require_gpu

pytestmark = pytest.mark.gpu

# (dtype, dk, dv): pipelined kernel first, then the generic kernel
PATHS = [(torch.bfloat16, 128, 128), (torch.bfloat16, 128, 64), (torch.bfloat16, 128, 16),
         (torch.bfloat16, 64, 64), (torch.float32, 64, 32), (torch.float32, 16, 16)]
IDS = ["bf16-128x128", "bf16-128x64", "bf16-128x16", "bf16-64x64", "f32-64x32", "f32-16x16"]


def _run(inp, g, init):
    dev = require_gpu()
    d = {k: v.to(dev) for k, v in inp.items()}
    gd = g.to(dev)
    o, S = la.deltanet_prefill(d["q"], d["k"], d["v"], d["beta"], g=gd,
                               S=d["S0"].clone() if init else None, use_initial_state=init)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.delta_recurrent(inp["q"], inp["k"], inp["v"], inp["beta"], g,
                                          S0=inp["S0"] if init else None)
    return (o, S), (o_ref, S_ref)


@pytest.mark.parametrize("init", [False, True], ids=["zero", "init"])
@pytest.mark.parametrize("per_token", [-3.0, -40.0], ids=["g-3", "g-40"])
@pytest.mark.parametrize("dtype,dk,dv", PATHS, ids=IDS)
def test_strong_decay_every_chunk(dtype, dk, dv, per_token, init):
    print(f"per-channel gate {per_token} per token, {dtype} dk={dk} dv={dv} init={init}", flush=True)
    inp = workloads.make_delta(2, 2, 150, dk, dv, dtype, seed=500 + dk + dv, init_state=init,
                               state_std=0.5)
    g = torch.full((2, 2, 150, dk), per_token).to(dtype)
    (o, S), (o_ref, S_ref) = _run(inp, g, init)
    assert_close(o, o_ref, TOL[dtype], "o")
    assert_close(S, S_ref, TOL[dtype], "S")


@pytest.mark.parametrize("dtype,dk,dv", PATHS, ids=IDS)
def test_burst_in_one_channel_of_one_chunk(dtype, dk, dv):
    """Mild decays everywhere (the workload's recipe) except channel 5 of
    tokens 70 .. 99, at -9 per token: only chunk 1 leaves the range."""
    print(f"per-channel gate burst, {dtype} dk={dk} dv={dv}", flush=True)
    inp = workloads.make_delta(1, 3, 200, dk, dv, dtype, seed=600 + dk + dv, gated=True,
                               init_state=True, state_std=0.5)
    g = inp.pop("g").clone()
    g[:, :, 70:100, 5] = -9.0
    (o, S), (o_ref, S_ref) = _run(inp, g, True)
    assert_close(o, o_ref, TOL[dtype], "o")
    assert_close(S, S_ref, TOL[dtype], "S")


@pytest.mark.parametrize("dtype,dk,dv", [PATHS[0], PATHS[4]], ids=[IDS[0], IDS[4]])
def test_growth(dtype, dk, dv):
    """g > 0 (a decay factor above 1): 1.1 per token in channel 3 of the
    second chunk (summed 70 > 64: out of range, while the values, about
    e^70, stay inside float32), 0.02 elsewhere."""
    print(f"per-channel gate growth, {dtype} dk={dk} dv={dv}", flush=True)
    inp = workloads.make_delta(1, 2, 128, dk, dv, dtype, seed=700 + dk, init_state=True,
                               state_std=0.1)
    g = torch.full((1, 2, 128, dk), 0.02)
    g[:, :, 64:, 3] = 1.1
    (o, S), (o_ref, S_ref) = _run(inp, g.to(dtype), True)
    assert_close(o, o_ref, TOL[dtype], "o")
    assert_close(S, S_ref, TOL[dtype], "S")
