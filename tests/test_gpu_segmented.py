"""deltanet_prefill_segmented (the sequence-parallel chunk-state scan) on the
GPU, through the C ABI, against the float64 oracle's per-token recurrence
over the whole sequence: the delta rule without a gate, with a decay per key
channel and with one decay per token; with and without an initial state;
segment lengths that are and are not whole chunks; every head-dimension
pair; the automatic segment count at a few-heads shape with a long sequence;
decays strong enough that every chunk leaves the factored form's range; and
the degenerate cases (one segment, no tokens, a split that does not divide
T, float32)."""
import pytest
import torch

import delta_rule_recurrent_chunkwise_amd as la
import oracle
import workloads
from gpu_common import TOL, assert_close, require_gpu

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
GATES = [None, "channel", "token"]
GEN_GATE = {None: False, "channel": True, "token": "token"}


def _run(inp, gate, P, init, what):
    dev = require_gpu()
    x = {n: t.to(dev) for n, t in inp.items()}
    S = x["S0"].clone() if init else None
    o, S = la.deltanet_prefill_segmented(x["q"], x["k"], x["v"], x["beta"], g=x.get("g"), gate=gate,
                                         S=S, use_initial_state=init, segments=P)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.delta_recurrent(inp["q"], inp["k"], inp["v"], inp["beta"], inp.get("g"),
                                          S0=inp["S0"] if init else None)
    assert_close(o, o_ref, TOL[BF16], f"o {what}")
    assert_close(S, S_ref, TOL[BF16], f"S {what}")
    return o, S


def _check(B, H, T, dk, dv, P, gate, init, seed, gscale=1.0):
    print(f"segmented prefill B={B} H={H} T={T} dk={dk} dv={dv} P={P} gate={gate} init={init}",
          flush=True)
    inp = workloads.make_delta(B, H, T, dk, dv, BF16, seed=seed, gated=GEN_GATE[gate],
                               init_state=init, state_std=0.5)
    if gscale != 1.0 and gate is not None:
        inp["g"] = (inp["g"].float() * gscale).to(BF16)
    return _run(inp, gate, P, init, f"T={T} P={P} gate={gate}")


@pytest.mark.parametrize("init", [False, True], ids=["zero", "init"])
@pytest.mark.parametrize("gate", GATES, ids=["no-gate", "per-channel", "per-token"])
@pytest.mark.parametrize("T,P", [(1024, 2), (1024, 4), (1024, 8), (960, 3), (1000, 8), (4096, 16)],
                         ids=["T1024-P2", "T1024-P4", "T1024-P8", "T960-P3", "T1000-P8", "T4096-P16"])
def test_segmented_equals_the_recurrence(T, P, gate, init):
    _check(1, 3, T, 128, 128, P, gate, init, 800 + T + P)


@pytest.mark.parametrize("gate", GATES, ids=["no-gate", "per-channel", "per-token"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (64, 64), (128, 16), (16, 128),
                                   (128, 64), (64, 128)])
def test_segmented_every_dim_pair(dk, dv, gate):
    """Dims other than 128 run the passes on the generic kernel (and d_v = 16
    the fix-up with one column tile); d_k = 16 pads the fix-up's 32-deep
    contraction with zeros."""
    _check(2, 2, 576, dk, dv, 6, gate, True, 900 + dk + 3 * dv)


def test_segmented_many_heads_and_batches():
    """B = 3, H = 5: segment-heads of different batches and heads interleave
    in the passes' view and in the scan's and fix-up's indexing."""
    _check(3, 5, 768, 128, 64, 4, "channel", True, 950)


@pytest.mark.parametrize("gate", GATES, ids=["no-gate", "per-channel", "per-token"])
def test_segmented_automatic_count_at_a_few_heads_long_sequence(gate):
    """B=1 H=4 T=32768 d=128, the shape the split is for: the library picks 16
    segments of 2048 tokens, and the whole output matches the recurrence."""
    assert la.deltanet_prefill_segments(1, 4, 32768, 128, 128) == 16
    _check(1, 4, 32768, 128, 128, 0, gate, True, 1000)


@pytest.mark.parametrize("gval", [-3.0, -40.0])
def test_segmented_strong_per_channel_decay(gval):
    """Every chunk's decay leaves the factored form's range: both passes walk
    them token by token, and the transitions are nearly zero."""
    inp = workloads.make_delta(1, 2, 640, 128, 128, BF16, seed=1100, gated=True, init_state=True,
                               state_std=0.5)
    inp["g"] = torch.full_like(inp["g"], gval)
    _run(inp, "channel", 5, True, f"g={gval}")


def test_segmented_burst_crossing_a_segment_boundary():
    """Strong decay in one channel over tokens 250 .. 270, across the boundary
    of segments 0 and 1 (256 tokens each): walked chunks on both sides."""
    inp = workloads.make_delta(1, 2, 1024, 128, 128, BF16, seed=1150, gated=True, init_state=True,
                               state_std=0.5)
    g = inp["g"].clone()
    g[:, :, 250:270, 7] = -9.0
    inp["g"] = g
    _run(inp, "channel", 4, True, "burst")


def test_one_segment_is_the_one_pass_entry_point():
    dev = require_gpu()
    inp = workloads.make_delta(2, 3, 300, 128, 128, BF16, seed=1200, gated=True, init_state=True,
                               state_std=0.5)
    x = {n: t.to(dev) for n, t in inp.items()}
    a = la.deltanet_prefill_segmented(x["q"], x["k"], x["v"], x["beta"], g=x["g"], gate="channel",
                                      S=x["S0"].clone(), use_initial_state=True, segments=1)
    b = la.deltanet_prefill(x["q"], x["k"], x["v"], x["beta"], g=x["g"], S=x["S0"].clone(),
                            use_initial_state=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_segmented_is_close_to_one_pass_at_the_few_heads_shape():
    """The split changes only the rounding: against the one-pass kernel at
    B=1 H=4 T=32768, per-token gate."""
    dev = require_gpu()
    inp = workloads.make_delta(1, 4, 32768, 128, 128, BF16, seed=1250, gated="token")
    x = {n: t.to(dev) for n, t in inp.items()}
    a = la.deltanet_prefill_segmented(x["q"], x["k"], x["v"], x["beta"], g=x["g"], gate="token")
    b = la.gated_deltanet_prefill(x["q"], x["k"], x["v"], x["beta"], x["g"])
    torch.cuda.synchronize()
    assert_close(a[0], b[0].float(), TOL[BF16], "o vs one pass")
    assert_close(a[1], b[1], TOL[BF16], "S vs one pass")


def test_segmented_repeated_calls_reuse_one_workspace():
    """The workspace's contents on entry do not matter: a second call on the
    same workspace, with other inputs and a smaller split, is exact too."""
    dev = require_gpu()
    ws = torch.empty(la.deltanet_prefill_segmented_workspace_bytes(None, 1, 2, 2048, 128, 128, BF16, 8),
                     device=dev, dtype=torch.uint8)
    for seed, P in ((1300, 8), (1301, 4)):
        inp = workloads.make_delta(1, 2, 2048, 128, 128, BF16, seed=seed, init_state=True,
                                   state_std=0.5)
        x = {n: t.to(dev) for n, t in inp.items()}
        o, S = la.deltanet_prefill_segmented(x["q"], x["k"], x["v"], x["beta"], S=x["S0"].clone(),
                                             use_initial_state=True, segments=P, workspace=ws)
        torch.cuda.synchronize()
        o_ref, S_ref = oracle.delta_recurrent(inp["q"], inp["k"], inp["v"], inp["beta"], None,
                                              S0=inp["S0"])
        assert_close(o, o_ref, TOL[BF16], f"o P={P}")
        assert_close(S, S_ref, TOL[BF16], f"S P={P}")


def test_segmented_empty_sequence_and_bad_splits():
    dev = require_gpu()
    e = torch.empty(1, 2, 0, 64, device=dev, dtype=BF16)
    eb = torch.empty(1, 2, 0, device=dev, dtype=BF16)
    S0 = torch.randn(1, 2, 64, 64, device=dev)
    _, S = la.deltanet_prefill_segmented(e, e, e, eb, S=S0.clone(), use_initial_state=True,
                                         segments=4)
    torch.cuda.synchronize()
    assert torch.equal(S, S0)
    inp = workloads.make_delta(1, 1, 100, 64, 64, BF16, seed=7)
    x = {n: t.to(dev) for n, t in inp.items()}
    with pytest.raises(la.LinAttnError):
        la.deltanet_prefill_segmented(x["q"], x["k"], x["v"], x["beta"], segments=3)
    f = {n: t.float() for n, t in x.items()}
    with pytest.raises(la.LinAttnError):
        la.deltanet_prefill_segmented(f["q"], f["k"], f["v"], f["beta"], segments=4)
