"""deltanet_prologue on the GPU against the float64 oracle: q, k =
normalize(silu(.)) (optionally scaled), beta = sigmoid(logits) with one logit
per token shared by the heads or one per head; in place; and followed by the
prefill, as the layer uses it."""
import math

import pytest
import torch

import delta_rule_recurrent_chunkwise_amd as la
import oracle
import workloads
from gpu_common import TOL, assert_close, require_gpu

pytestmark = pytest.mark.gpu


def _raw(B, H, T, dk, dtype, seed, bh):
    gen = workloads.generator(seed)
    q = (2.0 * torch.randn(B, H, T, dk, generator=gen)).to(dtype)
    k = (2.0 * torch.randn(B, H, T, dk, generator=gen)).to(dtype)
    lg = torch.randn(B, bh, T, generator=gen).to(dtype)
    return q, k, lg


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("dk", [16, 32, 64, 128])
@pytest.mark.parametrize("silu", [True, False], ids=["silu", "plain"])
@pytest.mark.parametrize("shared_beta", [True, False], ids=["beta1", "betaH"])
def test_prologue(dtype, dk, silu, shared_beta):
    dev = require_gpu()
    B, H, T = 2, 3, 100
    q, k, lg = _raw(B, H, T, dk, dtype, 900 + dk, 1 if shared_beta else H)
    scale = 1.0 / math.sqrt(dk)
    qo, ko, bo = la.deltanet_prologue(q.to(dev), k.to(dev), lg.to(dev), apply_silu=silu,
                                      q_scale=scale)
    torch.cuda.synchronize()
    assert_close(qo, oracle.qk_prologue(q, silu, scale), TOL[dtype], "q")
    assert_close(ko, oracle.qk_prologue(k, silu, 1.0), TOL[dtype], "k")
    assert_close(bo, oracle.beta_sigmoid(lg, H), TOL[dtype], "beta")


def test_prologue_in_place_and_zero_rows():
    """Outputs may overwrite the inputs; an all-zero row stays zero."""
    dev = require_gpu()
    q, k, _ = _raw(1, 2, 70, 64, torch.bfloat16, 5, 1)
    q[0, 1, 3] = 0
    qd, kd = q.to(dev), k.to(dev)
    la.deltanet_prologue(qd, kd, out=(qd, kd))
    torch.cuda.synchronize()
    assert_close(qd, oracle.qk_prologue(q, True, 1.0), 2e-2, "q in place")
    assert_close(kd, oracle.qk_prologue(k, True, 1.0), 2e-2, "k in place")
    assert torch.count_nonzero(qd[0, 1, 3]) == 0


def test_prologue_then_prefill_is_the_layer():
    """Raw q, k and one beta logit per token -> prologue -> deltanet_prefill
    equals the oracle's prologue followed by its recurrence."""
    dev = require_gpu()
    B, H, T, d = 2, 4, 192, 128
    q, k, lg = _raw(B, H, T, d, torch.bfloat16, 77, 1)
    gen = workloads.generator(78)
    v = torch.randn(B, H, T, d, generator=gen).to(torch.bfloat16)
    qo, ko, bo = la.deltanet_prologue(q.to(dev), k.to(dev), lg.to(dev))
    o, S = la.deltanet_prefill(qo, ko, v.to(dev), bo)
    torch.cuda.synchronize()
    qr = oracle.qk_prologue(q, True, 1.0)
    kr = oracle.qk_prologue(k, True, 1.0)
    br = oracle.beta_sigmoid(lg, H)
    o_ref, S_ref = oracle.delta_recurrent(qr, kr, v.double().numpy(), br)
    assert_close(o, o_ref, 2e-2, "o")
    assert_close(S, S_ref, 2e-2, "S")
