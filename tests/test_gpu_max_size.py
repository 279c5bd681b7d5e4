"""Tensors past 2^31 elements: every offset the kernels form must be 64-bit.

The inputs are a small seeded pool, tiled on the device. Heads never
interact and the kernels are deterministic, so every copy of a pool head
must come out bit for bit the same; an offset that wrapped would read or
write another copy's data and show up as a difference. The pool itself is
compared with the float64 oracle.

- across heads: B*H*T*d and the state B*H*dk*dv past 2^31 (one 64-token
  chunk per head, so about a million workgroups);
- within one head: T*d past 2^31 (over 2^24 tokens), with beta = 0 except
  on the last tokens, so the state stays exactly zero until then: every
  earlier output must be exactly 0, and the tail, read and written past
  2^31 elements, is compared with the oracle run from a zero state;
- decode: the state of N*H heads past 2^31 elements.
"""
import pytest
import torch

import delta_rule_recurrent_chunkwise_amd as la
import oracle
import workloads
from gpu_common import TOL, assert_close, require_gpu

pytestmark = pytest.mark.gpu

BF = torch.bfloat16
D = 128
POOL = 8  # distinct heads in the pool


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _same_copies(x, group):
    """Every copy of the first `group` heads (x viewed as [-1, group, ...])
    equals the first copy, bit for bit."""
    y = x.reshape(-1, group, *x.shape[-2:]) if x.dim() > 3 else x.reshape(-1, group, x.shape[-1])
    return bool(torch.equal(y, y[:1].expand_as(y)))


def test_prefill_past_2_31_elements_across_heads():
    dev = require_gpu()
    T = 64
    reps = 2**31 // (POOL * T * D) + 32
    n = reps * POOL * T * D
    print(f"deltanet_prefill across heads: B={reps} H={POOL} T={T} d={D}, {n} elements per token tensor", flush=True)
    assert n > 2**31 and reps * POOL * D * D > 2**31
    inp = workloads.make_delta(1, POOL, T, D, D, BF, seed=71)
    q, k, v, beta = (inp[x].to(dev).expand(reps, *inp[x].shape[1:]).contiguous() for x in ("q", "k", "v", "beta"))
    o, S = la.deltanet_prefill(q, k, v, beta)
    torch.cuda.synchronize()
    del q, k, v, beta
    assert _same_copies(o, POOL), "o differs between copies of one head"
    assert _same_copies(S, POOL), "S differs between copies of one head"
    o_ref, S_ref = oracle.delta_recurrent(inp["q"], inp["k"], inp["v"], inp["beta"])
    assert_close(o[-1:], o_ref, TOL[BF], "o (last batch, past 2^31 elements)")
    assert_close(S[-1:], S_ref, TOL[BF], "S (last batch, past 2^31 elements)")
    del o, S
    _free()


def test_prefill_past_2_31_elements_within_a_head():
    dev = require_gpu()
    T = 2**24 + 4096 + 37  # a ragged last chunk
    tail = 2 * 64 + 37      # tokens with beta != 0, from a chunk boundary on
    head = T - tail
    print(f"deltanet_prefill within one head: T={T} d={D}, {T * D} elements per token tensor", flush=True)
    assert head * D > 2**31 and head % 64 == 0  # the whole tail lies past 2^31 elements
    pool = workloads.make_delta(1, 1, 64, D, D, BF, seed=72)
    last = workloads.make_delta(1, 1, tail, D, D, BF, seed=73)
    ins = {}
    for x in ("q", "k", "v"):
        t = torch.empty(1, 1, T, D, dtype=BF, device=dev)
        t[0, 0, :head] = pool[x][0, 0].to(dev).unsqueeze(0).expand(head // 64, 64, D).reshape(head, D)
        t[0, 0, head:] = last[x][0, 0].to(dev)
        ins[x] = t
    beta = torch.zeros(1, 1, T, dtype=BF, device=dev)
    beta[0, 0, head:] = last["beta"][0, 0].to(dev)
    o, S = la.deltanet_prefill(ins["q"], ins["k"], ins["v"], beta)
    torch.cuda.synchronize()
    del ins, beta
    nz = int(torch.count_nonzero(o[0, 0, :head]))
    assert nz == 0, f"{nz} nonzero outputs where the state is exactly zero"
    o_ref, S_ref = oracle.delta_recurrent(last["q"], last["k"], last["v"], last["beta"])
    assert_close(o[:, :, head:], o_ref, TOL[BF], "o (tail, past 2^31 elements)")
    assert_close(S, S_ref, TOL[BF], "S after the tail")
    del o, S
    _free()


def test_decode_state_past_2_31_elements():
    dev = require_gpu()
    H = 32
    N = 2**31 // (H * D * D) + 4
    print(f"deltanet_decode_step: N={N} H={H} d={D}, state {N * H * D * D} elements", flush=True)
    assert N * H * D * D > 2**31 and (N * H) % POOL == 0
    inp = workloads.make_delta(1, POOL, 1, D, D, BF, seed=74, init_state=True)
    reps = N * H // POOL

    def tile(x, *shape):
        return x.to(dev).expand(reps, *x.shape[1:]).reshape(*shape).contiguous()

    q = tile(inp["q"][:, :, 0], N, H, D)
    k = tile(inp["k"][:, :, 0], N, H, D)
    v = tile(inp["v"][:, :, 0], N, H, D)
    beta = tile(inp["beta"][:, :, 0], N, H)
    S = tile(inp["S0"].float(), N, H, D, D)
    o = la.deltanet_decode_step(q, k, v, beta, S)
    torch.cuda.synchronize()
    del q, k, v, beta
    assert _same_copies(o, POOL), "o differs between copies of one head"
    assert _same_copies(S, POOL), "S differs between copies of one head"
    o_ref, S_ref = oracle.delta_recurrent(inp["q"], inp["k"], inp["v"], inp["beta"], S0=inp["S0"])
    assert_close(o.reshape(-1, POOL, D)[-1:], o_ref[:, :, 0], TOL[BF], "o (last heads, past 2^31 state elements)")
    assert_close(S.reshape(-1, POOL, D, D)[-1:], S_ref, TOL[BF], "S (last heads, past 2^31 elements)")
    del o, S
    _free()


# Grids: a launch's second and third dimensions are limited to 65535 blocks,
# so every count that grows with the input is in the first.

@pytest.mark.parametrize("gated", [False, True], ids=["la", "gla"])
def test_linear_attention_past_65535_heads(gated):
    """The chunk-parallel (bf16) linear-attention kernels over 65,600 heads of
    130 tokens (a ragged third chunk): the state scan runs one block row per
    head."""
    dev = require_gpu()
    d, T, reps = 16, 130, 8200
    print(f"{'gla' if gated else 'la'}_prefill: B={reps} H={POOL} T={T} d={d}", flush=True)
    assert reps * POOL > 65535
    if gated:
        inp = workloads.make_gla(1, POOL, T, d, d, BF, seed=75)
        names = ("q", "k", "v", "g")
    else:
        inp = workloads.make_la(1, POOL, T, d, d, BF, seed=75)
        names = ("q", "k", "v")
    x = {n: inp[n].to(dev).expand(reps, *inp[n].shape[1:]).contiguous() for n in names}
    if gated:
        o, S = la.gla_prefill(x["q"], x["k"], x["v"], x["g"])
        o_ref, S_ref = oracle.gla_recurrent(inp["q"], inp["k"], inp["v"], inp["g"])
    else:
        o, S, z = la.la_prefill(x["q"], x["k"], x["v"])
        o_ref, S_ref, z_ref = oracle.la_recurrent(inp["q"], inp["k"], inp["v"])
        assert _same_copies(z, POOL), "z differs between copies of one head"
        assert_close(z[-1:], z_ref, TOL[BF], "z (last batch)")
    torch.cuda.synchronize()
    assert _same_copies(o, POOL), "o differs between copies of one head"
    assert _same_copies(S, POOL), "S differs between copies of one head"
    assert_close(o[-1:], o_ref, TOL[BF], "o (last batch)")
    assert_close(S[-1:], S_ref, TOL[BF], "S (last batch)")
    del x, o, S
    _free()


def test_segmented_past_65535_fixup_blocks():
    """Two segments of 2^24 + 64 tokens each (d = 16): the output fix-up has
    65,537 blocks of 256 rows per segment.  beta = 0 except on the last chunk
    of each segment, so the state is exactly zero until the first of them,
    then the state S1 it leaves is carried unchanged to the second: every
    output of segment 0 before its last chunk is exactly 0, every output of
    segment 1 before its last chunk is q_t S1 (all 16.8 million compared),
    and the two active chunks follow the oracle."""
    dev = require_gpu()
    d, Tp = 16, 2**24 + 64
    T = 2 * Tp
    print(f"deltanet_prefill_segmented: T={T} in 2 segments, d={d}", flush=True)
    assert (Tp + 255) // 256 > 65535
    pool = workloads.make_delta(1, 1, 64, d, d, BF, seed=76)
    act = [workloads.make_delta(1, 1, 64, d, d, BF, seed=77 + i) for i in range(2)]
    ins = {}
    for n in ("q", "k", "v"):
        t = torch.empty(1, 1, T, d, dtype=BF, device=dev)
        for s in range(2):
            a0 = s * Tp
            t[0, 0, a0:a0 + Tp - 64] = pool[n][0, 0].to(dev).unsqueeze(0).expand((Tp - 64) // 64, 64, d).reshape(-1, d)
            t[0, 0, a0 + Tp - 64:a0 + Tp] = act[s][n][0, 0].to(dev)
        ins[n] = t
    beta = torch.zeros(1, 1, T, dtype=BF, device=dev)
    for s in range(2):
        beta[0, 0, (s + 1) * Tp - 64:(s + 1) * Tp] = act[s]["beta"][0, 0].to(dev)
    o, S = la.deltanet_prefill_segmented(ins["q"], ins["k"], ins["v"], beta, segments=2)
    torch.cuda.synchronize()
    o0_ref, S1 = oracle.delta_recurrent(act[0]["q"], act[0]["k"], act[0]["v"], act[0]["beta"])
    o1_ref, S_ref = oracle.delta_recurrent(act[1]["q"], act[1]["k"], act[1]["v"], act[1]["beta"], S0=S1)
    nz = int(torch.count_nonzero(o[0, 0, :Tp - 64]))
    assert nz == 0, f"{nz} nonzero outputs where the state is exactly zero"
    assert_close(o[:, :, Tp - 64:Tp], o0_ref, TOL[BF], "o (segment 0, last chunk)")
    S1d = torch.as_tensor(S1, dtype=torch.float32).reshape(d, d).to(dev)
    ref = ins["q"][0, 0, Tp:T - 64].float() @ S1d
    err = float((o[0, 0, Tp:T - 64].float() - ref).abs().max() / ref.abs().max())
    print(f"  o (segment 1, {Tp - 64} tokens against q S1): rel err {err:.3e} (tol {TOL[BF]:g})", flush=True)
    assert err <= TOL[BF]
    assert_close(o[:, :, T - 64:], o1_ref, TOL[BF], "o (segment 1, last chunk)")
    assert_close(S, S_ref, TOL[BF], "S")
    del ins, beta, o, S, ref
    _free()


@pytest.mark.parametrize("gate", ["channel", "token"])
def test_gated_prefill_past_2_31_elements_across_heads(gate):
    """The gated prefills over more than 2^31 elements per token tensor: a
    decay per key channel (its pre-pass writes three scaled copies of q and k
    into the workspace) and one per token."""
    dev = require_gpu()
    T = 64
    reps = 2**31 // (POOL * T * D) + 32
    print(f"gated prefill ({gate}) across heads: B={reps} H={POOL} T={T} d={D}", flush=True)
    inp = workloads.make_delta(1, POOL, T, D, D, BF, seed=79, gated=True if gate == "channel" else "token")
    x = {n: inp[n].to(dev).expand(reps, *inp[n].shape[1:]).contiguous() for n in ("q", "k", "v", "beta", "g")}
    assert x["q"].numel() > 2**31
    if gate == "channel":
        o, S = la.deltanet_prefill(x["q"], x["k"], x["v"], x["beta"], g=x["g"])
    else:
        o, S = la.gated_deltanet_prefill(x["q"], x["k"], x["v"], x["beta"], x["g"])
    torch.cuda.synchronize()
    del x
    assert _same_copies(o, POOL), "o differs between copies of one head"
    assert _same_copies(S, POOL), "S differs between copies of one head"
    o_ref, S_ref = oracle.delta_recurrent(inp["q"], inp["k"], inp["v"], inp["beta"], g=inp["g"])
    assert_close(o[-1:], o_ref, TOL[BF], "o (last batch, past 2^31 elements)")
    assert_close(S[-1:], S_ref, TOL[BF], "S (last batch, past 2^31 elements)")
    del o, S
    _free()


def test_backward_past_2_31_elements_across_heads():
    """deltanet_prefill_backward over more than 2^31 elements per token
    tensor (its workspace holds the chunk states, P, R^T and dSn of about a
    million chunks): every copy of a pool head gets the same gradients, and
    the pool's gradients follow the oracle's reverse recurrence."""
    dev = require_gpu()
    T = 64
    reps = 2**31 // (POOL * T * D) + 32
    print(f"deltanet_prefill_backward across heads: B={reps} H={POOL} T={T} d={D}", flush=True)
    inp = workloads.make_delta(1, POOL, T, D, D, BF, seed=80)
    dO = torch.randn(1, POOL, T, D, generator=workloads.generator(81)).to(BF)
    x = {n: inp[n].to(dev).expand(reps, *inp[n].shape[1:]).contiguous() for n in ("q", "k", "v", "beta")}
    dOd = dO.to(dev).expand(reps, POOL, T, D).contiguous()
    assert dOd.numel() > 2**31
    grads = la.deltanet_prefill_backward(x["q"], x["k"], x["v"], x["beta"], dOd)
    torch.cuda.synchronize()
    del x, dOd
    ref = oracle.delta_backward(inp["q"], inp["k"], inp["v"], inp["beta"], dO)
    for name, g, r in zip(("dq", "dk", "dv", "dbeta"), grads, ref):
        if g.dim() == 3:
            assert bool(torch.equal(g, g[:1].expand_as(g))), f"{name} differs between copies of one head"
        else:
            assert _same_copies(g, POOL), f"{name} differs between copies of one head"
        assert_close(g[-1:], r, TOL[BF], f"{name} (last batch, past 2^31 elements)")
    del grads
    _free()
