"""The identity behind the sequence-parallel chunk-state scan, checked with the
oracle alone (CPU): the delta rule run as P segments, each from zero and from
the identity with v = 0, then the incoming states scanned and the outputs
corrected, equals one run over the whole sequence.  The state update is affine
in the state (article "From GPT-2 to Kimi K3, explained", section "DeltaNet
(Parallelizing Linear Transformers with Delta Rule)": every chunk starts from
the previous chunk's final state), with or without a decay ("Gated Delta
Net", "KDA / Kimi Linear")."""
import numpy as np
import pytest
import torch

import oracle
import workloads


def _segments(x, B, H, P, Tp):
    return x.reshape(B, H * P, Tp, *x.shape[3:]).contiguous()


@pytest.mark.parametrize("gated", [False, True, "token"], ids=["no-gate", "per-channel", "per-token"])
@pytest.mark.parametrize("init", [False, True], ids=["zero", "init"])
def test_segment_scan_equals_one_pass(gated, init):
    B, H, T, dk, dv, P = 1, 2, 96, 16, 8, 3
    Tp = T // P
    inp = workloads.make_delta(B, H, T, dk, dv, torch.float32, seed=31, gated=gated,
                               init_state=init, state_std=0.5)
    q, k, v, beta = (inp[n] for n in ("q", "k", "v", "beta"))
    g = inp.get("g")
    S0 = inp["S0"] if init else None
    o_ref, S_ref = oracle.delta_recurrent(q, k, v, beta, g, S0=S0)

    qs, ks, vs = (_segments(x, B, H, P, Tp) for x in (q, k, v))
    bs = beta.reshape(B, H * P, Tp).contiguous()
    gs = None if g is None else _segments(g, B, H, P, Tp)
    # each segment from zero, and each segment's transition (from I, v = 0)
    o0, Sz = oracle.delta_recurrent(qs, ks, vs, bs, gs)
    eye = torch.eye(dk, dtype=torch.float32).expand(B, H * P, dk, dk).contiguous()
    oB, M = oracle.delta_recurrent(qs, ks, torch.zeros(B, H * P, Tp, dk), bs, gs, S0=eye)
    o0 = o0.reshape(B, H, P, Tp, dv)
    Sz = Sz.reshape(B, H, P, dk, dv)
    oB = oB.reshape(B, H, P, Tp, dk)
    M = M.reshape(B, H, P, dk, dk)
    Sin = np.zeros((B, H, P, dk, dv))
    if init:
        Sin[:, :, 0] = S0.double().numpy()
    for p in range(1, P):
        Sin[:, :, p] = M[:, :, p - 1] @ Sin[:, :, p - 1] + Sz[:, :, p - 1]
    S = M[:, :, P - 1] @ Sin[:, :, P - 1] + Sz[:, :, P - 1]
    o = (o0 + oB @ Sin).reshape(B, H, T, dv)
    scale = np.abs(o_ref).max()
    assert np.abs(o - o_ref).max() <= 1e-12 * scale * T
    assert np.abs(S - S_ref).max() <= 1e-12 * np.abs(S_ref).max() * T
