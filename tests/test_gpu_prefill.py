"""Chunkwise prefill on the GPU against the float64 oracle, through the C ABI,
at sizes the oracle finishes in seconds that still span several 64-token
chunks, plus the method's special cases and cross-entry-point checks."""
import numpy as np
import pytest
import torch

import delta_rule_recurrent_chunkwise_amd as la
import oracle
import workloads
from gpu_common import TOL, assert_close, rel_err, require_gpu

pytestmark = pytest.mark.gpu

DIMS = [(16, 16), (32, 64), (64, 32), (64, 64), (128, 128), (128, 16), (16, 128)]
DTYPES = [torch.float32, torch.bfloat16]
IDS = ["f32", "bf16"]


def _dev(d, dev):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def _run_delta(inp, dev, gated, init):
    d = _dev(inp, dev)
    S = d["S0"].clone() if init else None
    o, S = la.deltanet_prefill(d["q"], d["k"], d["v"], d["beta"], g=d.get("g"), S=S,
                               use_initial_state=init)
    torch.cuda.synchronize()
    return o, S


@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
@pytest.mark.parametrize("dk,dv", DIMS)
@pytest.mark.parametrize("gated", [False, True], ids=["delta", "gated"])
@pytest.mark.parametrize("init", [False, True], ids=["zero", "init"])
def test_deltanet_prefill(dtype, dk, dv, gated, init):
    dev = require_gpu()
    if gated and dtype == torch.float32 and dk > 64:
        pytest.skip("float32 gated prefill supports dk <= 64 (LDS footprint)")
    B, H, T = 2, 3, 192
    inp = workloads.make_delta(B, H, T, dk, dv, dtype, seed=100 + dk + 3 * dv,
                               gated=gated, init_state=init, state_std=0.5)
    o, S = _run_delta(inp, dev, gated, init)
    o_ref, S_ref = oracle.delta_recurrent(inp["q"], inp["k"], inp["v"], inp["beta"],
                                          inp.get("g"), S0=inp["S0"] if init else None)
    assert_close(o, o_ref, TOL[dtype], "o")
    assert_close(S, S_ref, TOL[dtype], "S")


@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
@pytest.mark.parametrize("dk,dv", DIMS)
@pytest.mark.parametrize("init", [False, True], ids=["zero", "init"])
def test_la_prefill(dtype, dk, dv, init):
    dev = require_gpu()
    B, H, T = 2, 3, 192
    inp = workloads.make_la(B, H, T, dk, dv, dtype, seed=200 + dk + 3 * dv, init_state=init)
    d = _dev(inp, dev)
    S = d["S0"].clone() if init else None
    z = d["z0"].clone() if init else None
    o, S, z = la.la_prefill(d["q"], d["k"], d["v"], S=S, z=z, use_initial_state=init)
    torch.cuda.synchronize()
    o_ref, S_ref, z_ref = oracle.la_recurrent(inp["q"], inp["k"], inp["v"],
                                              inp["S0"] if init else None,
                                              inp["z0"] if init else None)
    assert_close(o, o_ref, TOL[dtype], "o")
    assert_close(S, S_ref, TOL[dtype], "S")
    assert_close(z, z_ref, TOL[dtype], "z")


@pytest.mark.parametrize("gated", [False, True], ids=["delta", "gated"])
def test_many_heads_bf16_dk128(gated):
    """Enough (batch, head) pairs that the bf16 dk = 128 kernels take their
    32-column value slices (few pairs select 16-column slices)."""
    dev = require_gpu()
    B, H, T = 8, 32, 128
    inp = workloads.make_delta(B, H, T, 128, 128, torch.bfloat16, seed=321, gated=gated,
                               init_state=True, state_std=0.5)
    o, S = _run_delta(inp, dev, gated, True)
    o_ref, S_ref = oracle.delta_recurrent(inp["q"], inp["k"], inp["v"], inp["beta"],
                                          inp.get("g"), S0=inp["S0"])
    assert_close(o, o_ref, TOL[torch.bfloat16], "o")
    assert_close(S, S_ref, TOL[torch.bfloat16], "S")


def test_float32_gated_dk128_is_rejected():
    dev = require_gpu()
    inp = workloads.make_delta(1, 1, 64, 128, 64, torch.float32, seed=1, gated=True)
    d = _dev(inp, dev)
    with pytest.raises(la.LinAttnError) as e:
        la.deltanet_prefill(d["q"], d["k"], d["v"], d["beta"], g=d["g"])
    assert e.value.code == -4


@pytest.mark.parametrize("gated", [False, True], ids=["delta", "gated"])
def test_short_and_long_sequences(gated):
    """T = 64, 128, 320 and 1024 (1, 2, 5 and 16 chunks), bf16, d = 128: the
    pipelined kernel's loop runs its bodies in pairs with an odd one after,
    and its loaders start one or two chunks ahead."""
    dev = require_gpu()
    for T in (64, 128, 320, 1024):
        inp = workloads.make_delta(1, 2, T, 128, 128, torch.bfloat16, seed=T + gated, gated=gated)
        o, S = _run_delta(inp, dev, gated, False)
        o_ref, S_ref = oracle.delta_recurrent(inp["q"], inp["k"], inp["v"], inp["beta"],
                                              inp.get("g"))
        assert_close(o, o_ref, 2e-2, f"o T={T}")
        assert_close(S, S_ref, 2e-2, f"S T={T}")


RAGGED_T = (1, 63, 65, 100, 130)


@pytest.mark.parametrize("mode", ["la", "delta", "gated"])
@pytest.mark.parametrize("dtype,dk,dv", [(torch.bfloat16, 128, 128), (torch.bfloat16, 64, 32),
                                         (torch.float32, 64, 64)],
                         ids=["bf16-128x128", "bf16-64x32", "f32-64x64"])
def test_ragged_lengths(mode, dtype, dk, dv):
    """T not a multiple of 64 (a partial last chunk, or one chunk of one
    token) in every prefill kernel: bf16 d = 128 takes the pipelined delta
    kernels and the chunk-parallel linear attention, the others the generic
    kernel.  Odd T starts from an initial state."""
    dev = require_gpu()
    for T in RAGGED_T:
        init = T % 2 == 1
        seed = 1000 + T + 7 * dk + dv
        print(f"  mode={mode} T={T} init={init}", flush=True)
        if mode == "la":
            inp = workloads.make_la(2, 3, T, dk, dv, dtype, seed=seed, init_state=init)
            d = _dev(inp, dev)
            o, S, z = la.la_prefill(d["q"], d["k"], d["v"], S=d["S0"].clone() if init else None,
                                    z=d["z0"].clone() if init else None, use_initial_state=init)
            torch.cuda.synchronize()
            o_ref, S_ref, z_ref = oracle.la_recurrent(inp["q"], inp["k"], inp["v"],
                                                      inp["S0"] if init else None,
                                                      inp["z0"] if init else None)
            assert_close(z, z_ref, TOL[dtype], f"z T={T}")
        else:
            inp = workloads.make_delta(2, 3, T, dk, dv, dtype, seed=seed, gated=mode == "gated",
                                       init_state=init, state_std=0.5)
            o, S = _run_delta(inp, dev, mode == "gated", init)
            o_ref, S_ref = oracle.delta_recurrent(inp["q"], inp["k"], inp["v"], inp["beta"],
                                                  inp.get("g"), S0=inp["S0"] if init else None)
        assert tuple(o.shape) == (2, 3, T, dv)
        assert_close(o, o_ref, TOL[dtype], f"o T={T}")
        assert_close(S, S_ref, TOL[dtype], f"S T={T}")


@pytest.mark.parametrize("gated", [False, True], ids=["delta", "gated"])
def test_ragged_many_heads_bf16_dk128(gated):
    """A partial last chunk with 32-column value slices (many (batch, head)
    pairs), where the output tile of the last chunk is written by the store
    after the loop."""
    dev = require_gpu()
    inp = workloads.make_delta(8, 32, 100, 128, 128, torch.bfloat16, seed=77, gated=gated,
                               init_state=True, state_std=0.5)
    o, S = _run_delta(inp, dev, gated, True)
    o_ref, S_ref = oracle.delta_recurrent(inp["q"], inp["k"], inp["v"], inp["beta"],
                                          inp.get("g"), S0=inp["S0"])
    assert_close(o, o_ref, TOL[torch.bfloat16], "o")
    assert_close(S, S_ref, TOL[torch.bfloat16], "S")


def test_partial_chunk_leaves_memory_past_the_end_alone():
    """The output rows of a partial chunk that do not exist are never
    written: o is a view into a larger buffer whose next row holds a
    sentinel."""
    dev = require_gpu()
    T, dv = 100, 128
    inp = workloads.make_delta(1, 1, T, 128, dv, torch.bfloat16, seed=5)
    d = _dev(inp, dev)
    buf = torch.full((T + 28, dv), 7.0, device=dev, dtype=torch.bfloat16)
    o = buf[:T].view(1, 1, T, dv)
    la.deltanet_prefill(d["q"], d["k"], d["v"], d["beta"], o=o)
    torch.cuda.synchronize()
    assert torch.all(buf[T:] == 7.0)
    o_ref, _ = oracle.delta_recurrent(inp["q"], inp["k"], inp["v"], inp["beta"])
    assert_close(o, o_ref, TOL[torch.bfloat16], "o")


@pytest.mark.parametrize("mode", ["la", "delta", "gated"])
@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
def test_empty_sequence(mode, dtype):
    """T = 0: the final state is the initial state when one is given, and
    zero otherwise (the sum over no tokens); the output is empty."""
    dev = require_gpu()
    B, H, dk, dv = 2, 3, 64, 32
    gen = torch.Generator().manual_seed(9)
    S0 = torch.randn(B, H, dk, dv, generator=gen).to(dev)
    z0 = torch.rand(B, H, dk, generator=gen).to(dev) + 1.0
    e = torch.empty(B, H, 0, dk, device=dev, dtype=dtype)
    ev = torch.empty(B, H, 0, dv, device=dev, dtype=dtype)
    eb = torch.empty(B, H, 0, device=dev, dtype=dtype)
    for init in (True, False):
        S = S0.clone()
        if mode == "la":
            z = z0.clone()
            o, S, z = la.la_prefill(e, e, ev, S=S, z=z, use_initial_state=init)
            torch.cuda.synchronize()
            assert torch.equal(z, z0 if init else torch.zeros_like(z0))
        else:
            o, S = la.deltanet_prefill(e, e, ev, eb, g=e if mode == "gated" else None, S=S,
                                       use_initial_state=init)
            torch.cuda.synchronize()
        assert tuple(o.shape) == (B, H, 0, dv)
        assert torch.equal(S, S0 if init else torch.zeros_like(S0))


def test_beta_zero_keeps_state_and_reads_it():
    dev = require_gpu()
    inp = workloads.make_delta(1, 2, 128, 64, 64, torch.float32, seed=3, init_state=True,
                               state_std=1.0)
    inp["beta"] = torch.zeros_like(inp["beta"])
    o, S = _run_delta(inp, dev, False, True)
    assert_close(S, inp["S0"], 1e-6, "S unchanged")
    ref = torch.einsum("bhtd,bhde->bhte", inp["q"].double(), inp["S0"].double())
    assert_close(o, ref, 1e-5, "o = q S0")


def test_exact_retrieval_with_orthonormal_keys():
    """beta = 1, orthonormal keys, zero state: K S_T = V and a query equal to an
    earlier key reads back that key's value (fp32 inputs)."""
    dev = require_gpu()
    d, T = 128, 128
    gen = torch.Generator().manual_seed(9)
    Qm, _ = torch.linalg.qr(torch.randn(d, d, generator=gen, dtype=torch.float64))
    keys = Qm.T[:T // 2].float()                    # 64 orthonormal rows
    k = torch.cat([keys, keys.flip(0)])[None, None].contiguous()   # rewrite in reverse
    v = torch.randn(1, 1, T, d, generator=gen)
    q = k.clone()
    beta = torch.ones(1, 1, T)
    o, S = la.deltanet_prefill(q.to(dev), k.to(dev), v.to(dev), beta.to(dev))
    torch.cuda.synchronize()
    # the second half rewrites every key: it must read back the newest value
    assert_close(o[0, 0], v[0, 0], 1e-4, "o_t = v_t")
    newest = v[0, 0, T // 2:].flip(0)               # value now stored at keys[i]
    assert_close(keys.to(dev) @ S[0, 0], newest, 1e-4, "K S = newest V")


def test_gate_limits():
    """g = 0 equals the ungated rule; a strong uniform decay (a = e^-1.2 per
    token, a cumulative log-decay of -76.8 over a 64-token chunk, near the
    range the chunk form supports) still matches the oracle."""
    dev = require_gpu()
    inp = workloads.make_delta(1, 2, 128, 64, 64, torch.bfloat16, seed=4, gated=True,
                               init_state=True)
    o1, S1 = _run_delta(dict(inp, g=torch.zeros_like(inp["g"])), dev, True, True)
    plain = {k: v for k, v in inp.items() if k != "g"}
    o2, S2 = _run_delta(plain, dev, False, True)
    assert_close(o1, o2.float(), 1e-6, "g=0 vs ungated o")
    assert_close(S1, S2, 1e-6, "g=0 vs ungated S")
    strong = dict(inp, g=torch.full_like(inp["g"], -1.2))
    o3, S3 = _run_delta(strong, dev, True, True)
    o_ref, S_ref = oracle.delta_recurrent(strong["q"], strong["k"], strong["v"],
                                          strong["beta"], strong["g"], S0=strong["S0"])
    assert_close(o3, o_ref, 2e-2, "strong decay o")
    assert_close(S3, S_ref, 2e-2, "strong decay S")


def test_decode_gate_clears_memory():
    """Decode with a very negative log-decay: the state is cleared before the
    write, so S = beta k^T v and o = beta (q.k) v."""
    dev = require_gpu()
    inp = workloads.make_decode(3, 2, 64, 32, torch.float32, seed=6, gated=True, ring=1)
    S = inp["S0"].to(dev)
    g = torch.full_like(inp["g"][0], -200.0)
    q, k, v, beta = (inp[n][0] for n in ("q", "k", "v", "beta"))
    o = la.deltanet_decode_step(q.to(dev), k.to(dev), v.to(dev), beta.to(dev), S, g=g.to(dev))
    torch.cuda.synchronize()
    ref_S = beta.double()[..., None, None] * k.double()[..., :, None] * v.double()[..., None, :]
    ref_o = (beta.double() * (q.double() * k.double()).sum(-1))[..., None] * v.double()
    assert_close(S, ref_S, 1e-5, "cleared S")
    assert_close(o, ref_o, 1e-4, "cleared o")


@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
def test_split_prefill_equals_full(dtype):
    """prefill(T1) then prefill(T2) from the returned state equals prefill(T1+T2)
    exactly (same chunks, fp32 state carried through memory)."""
    dev = require_gpu()
    inp = workloads.make_delta(2, 2, 256, 64, 128, dtype, seed=12, gated=True)
    if dtype == torch.float32:
        inp = workloads.make_delta(2, 2, 256, 64, 64, dtype, seed=12, gated=True)
    d = _dev(inp, dev)
    o, S = la.deltanet_prefill(d["q"], d["k"], d["v"], d["beta"], g=d["g"])
    cut = 128
    part = {n: d[n][:, :, :cut].contiguous() for n in ("q", "k", "v", "beta", "g")}
    rest = {n: d[n][:, :, cut:].contiguous() for n in ("q", "k", "v", "beta", "g")}
    o1, S1 = la.deltanet_prefill(part["q"], part["k"], part["v"], part["beta"], g=part["g"])
    o2, S2 = la.deltanet_prefill(rest["q"], rest["k"], rest["v"], rest["beta"], g=rest["g"],
                                 S=S1, use_initial_state=True)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2], dim=2), o)
    assert torch.equal(S2, S)
    la_inp = _dev(workloads.make_la(1, 2, 192, 32, 32, dtype, seed=13), dev)
    oa, Sa, za = la.la_prefill(la_inp["q"], la_inp["k"], la_inp["v"])
    c = {n: la_inp[n][:, :, :64].contiguous() for n in ("q", "k", "v")}
    r = {n: la_inp[n][:, :, 64:].contiguous() for n in ("q", "k", "v")}
    ob1, Sb1, zb1 = la.la_prefill(c["q"], c["k"], c["v"])
    ob2, Sb2, zb2 = la.la_prefill(r["q"], r["k"], r["v"], S=Sb1, z=zb1, use_initial_state=True)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([ob1, ob2], dim=2), oa)
    assert torch.equal(Sb2, Sa) and torch.equal(zb2, za)


@pytest.mark.parametrize("gated", [False, True], ids=["delta", "gated"])
def test_prefill_equals_decode_steps(gated):
    """The chunkwise prefill and T one-token decode steps compute the same
    recurrence (GPU against GPU, fp32)."""
    dev = require_gpu()
    B, H, T, dk, dv = 1, 3, 128, 32, 64
    inp = _dev(workloads.make_delta(B, H, T, dk, dv, torch.float32, seed=21, gated=gated,
                                    init_state=True, state_std=0.3), dev)
    o, S = la.deltanet_prefill(inp["q"], inp["k"], inp["v"], inp["beta"], g=inp.get("g"),
                               S=inp["S0"].clone(), use_initial_state=True)
    Sd = inp["S0"].clone()
    outs = []
    for t in range(T):
        sl = {n: inp[n][:, :, t].contiguous() for n in ("q", "k", "v", "beta")}
        g = inp["g"][:, :, t].contiguous() if gated else None
        outs.append(la.deltanet_decode_step(sl["q"], sl["k"], sl["v"], sl["beta"], Sd, g=g))
    torch.cuda.synchronize()
    assert_close(o, torch.stack(outs, dim=2), 1e-4, "prefill vs decode o")
    assert_close(S, Sd, 1e-4, "prefill vs decode S")


def test_la_prefill_equals_decode_steps():
    dev = require_gpu()
    B, H, T, d = 1, 2, 128, 32
    inp = _dev(workloads.make_la(B, H, T, d, d, torch.float32, seed=22, init_state=True), dev)
    o, S, z = la.la_prefill(inp["q"], inp["k"], inp["v"], S=inp["S0"].clone(),
                            z=inp["z0"].clone(), use_initial_state=True)
    Sd, zd = inp["S0"].clone(), inp["z0"].clone()
    outs = [la.la_decode_step(inp["q"][:, :, t].contiguous(), inp["k"][:, :, t].contiguous(),
                              inp["v"][:, :, t].contiguous(), Sd, zd) for t in range(T)]
    torch.cuda.synchronize()
    assert_close(o, torch.stack(outs, dim=2), 1e-4, "la prefill vs decode o")
    assert_close(S, Sd, 1e-4, "la prefill vs decode S")
    assert_close(z, zd, 1e-5, "la prefill vs decode z")


def test_deterministic():
    dev = require_gpu()
    inp = _dev(workloads.make_delta(2, 4, 512, 128, 128, torch.bfloat16, seed=31,
                                    gated=True), dev)
    a = la.deltanet_prefill(inp["q"], inp["k"], inp["v"], inp["beta"], g=inp["g"])
    b = la.deltanet_prefill(inp["q"], inp["k"], inp["v"], inp["beta"], g=inp["g"])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_nan_stays_in_its_head():
    """A NaN in one token of one head poisons that head from the token's chunk
    on; every other head still matches the oracle."""
    dev = require_gpu()
    B, H, T, d = 1, 4, 192, 64
    inp = workloads.make_delta(B, H, T, d, d, torch.bfloat16, seed=41)
    inp["v"][0, 2, 100, 5] = float("nan")
    o, S = _run_delta(inp, dev, False, False)
    o_ref, S_ref = oracle.delta_recurrent(inp["q"], inp["k"], inp["v"], inp["beta"])
    ok = [0, 1, 3]
    assert_close(o[:, ok], o_ref[:, ok], 2e-2, "clean heads o")
    assert_close(S[:, ok], S_ref[:, ok], 2e-2, "clean heads S")
    oc = o[0, 2].float().cpu()
    assert torch.isfinite(oc[:64]).all(), "chunks before the NaN stay finite"
    assert torch.isnan(oc[128:]).any(axis=1).all(), "NaN reaches every later token"
    assert torch.isnan(S[0, 2]).any()
