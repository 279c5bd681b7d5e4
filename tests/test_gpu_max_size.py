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
