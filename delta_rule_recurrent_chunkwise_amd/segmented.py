"""Sequence-parallel chunk-state scan for the delta rule: a measured prototype.

With the tokens fixed, one step of the delta rule,
S <- (I - beta k k^T) diag(a) S + beta k v^T, is affine in the state S, and so
is any run of steps: S_out = M S_in + S_zero, where M (d_k x d_k) is the
product of the steps' linear parts and S_zero is the state reached from zero.
Each output is linear in the incoming state as well:
o_t = o_t(from zero) + S_in^T (M_t^T q_t), with M_t the product up to token t.
(Article "From GPT-2 to Kimi K3, explained", section "DeltaNet (Parallelizing
Linear Transformers with Delta Rule)": each chunk continues from the state the
previous one left; "Gated Delta Net" and "KDA / Kimi Linear" for the decays.)

So a long sequence can be cut into P segments that are processed at once:

1. every segment from a zero state: its outputs o0 and final state S_zero;
2. every segment from the identity (d_v = d_k) with v = 0: its final state is
   M, and its outputs are the rows M_t^T q_t;
3. the segments' incoming states by a scan over the segments:
   S_in[0] = S0, S_in[p] = M[p-1] S_in[p-1] + S_zero[p-1];
4. o = o0 + (M_t^T q_t)^T S_in per segment; the final state is
   M[P-1] S_in[P-1] + S_zero[P-1].

Steps 1 and 2 call the library's prefill entry points on a view of the inputs
in which the segments are extra heads ([B, H, T, d] read as [B, H*P, T/P, d],
no copy). Steps 3 and 4 are torch matrix products. This module exists to
measure that composition against the one-pass kernel at the same shapes; it
is not an entry point of the library, and nothing in the library calls it.
"""
from __future__ import annotations

import torch

from . import deltanet_prefill, deltanet_prefill_workspace_bytes, gated_deltanet_prefill


class SegmentBuffers:
    """Every buffer the segmented prefill writes, allocated once for one
    shape so that repeated calls allocate nothing."""

    def __init__(self, B, H, T, dk, dv, segments, dtype, device, gated):
        P = segments
        if T % P:
            raise ValueError(f"T = {T} is not a multiple of the segment count {P}")
        Tp, HP = T // P, H * P
        self.shape = (B, H, T, dk, dv, P)
        self.o0 = torch.empty(B, HP, Tp, dv, device=device, dtype=dtype)
        self.oB = torch.empty(B, HP, Tp, dk, device=device, dtype=dtype)
        self.Sz = torch.empty(B, HP, dk, dv, device=device, dtype=torch.float32)
        self.M = torch.empty(B, HP, dk, dk, device=device, dtype=torch.float32)
        self.eye = torch.eye(dk, device=device, dtype=torch.float32).expand(B, HP, dk, dk).contiguous()
        self.vzero = torch.zeros(B, HP, Tp, dk, device=device, dtype=dtype)
        self.Sin = torch.empty(B, H, P, dk, dv, device=device, dtype=torch.float32)
        self.S = torch.empty(B, H, dk, dv, device=device, dtype=torch.float32)
        nbytes = deltanet_prefill_workspace_bytes(gated, B, HP, Tp, dk, max(dk, dv), dtype)
        self.ws = torch.empty(max(nbytes, 1), device=device, dtype=torch.uint8)


def segmented_delta_prefill(q, k, v, beta, segments, g=None, token_gate=False, S0=None,
                            buffers=None, stream=None, timer=None):
    """The delta rule over q, k [B,H,T,dk], v [B,H,T,dv], beta [B,H,T] (and
    g: [B,H,T,dk] per key channel, or [B,H,T] with token_gate) computed as
    `segments` segments of T / segments tokens each, as described above.
    Returns (o [B,H,T,dv], S [B,H,dk,dv] fp32); o and S live in `buffers`.
    `timer(name)`, if given, is called after each of the four steps is
    enqueued (the bench records an event there)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    P = segments
    buf = buffers or SegmentBuffers(B, H, T, dk, dv, P, q.dtype, q.device,
                                    g is not None and not token_gate)
    if buf.shape != (B, H, T, dk, dv, P):
        raise ValueError("buffers were made for another shape")
    Tp, HP = T // P, H * P
    qs, ks, vs = (x.view(B, HP, Tp, x.shape[-1]) for x in (q, k, v))
    bs = beta.view(B, HP, Tp)
    if g is None:
        gs = None
    else:
        gs = g.view(B, HP, Tp) if token_gate else g.view(B, HP, Tp, dk)

    def run(vv, S, o, init):
        if token_gate:
            gated_deltanet_prefill(qs, ks, vv, bs, gs, S=S, use_initial_state=init, o=o,
                                   stream=stream)
        else:
            deltanet_prefill(qs, ks, vv, bs, g=gs, S=S, use_initial_state=init, o=o,
                             stream=stream, workspace=buf.ws)

    # 1. each segment from zero
    run(vs, buf.Sz, buf.o0, False)
    if timer:
        timer("segments_from_zero")
    # 2. each segment's transition (from the identity, v = 0)
    buf.M.copy_(buf.eye)
    run(buf.vzero, buf.M, buf.oB, True)
    if timer:
        timer("transitions")
    # 3. scan over the segments
    M = buf.M.view(B, H, P, dk, dk)
    Sz = buf.Sz.view(B, H, P, dk, dv)
    Sin = buf.Sin
    if S0 is None:
        Sin[:, :, 0].zero_()
    else:
        Sin[:, :, 0].copy_(S0)
    for p in range(1, P):
        torch.matmul(M[:, :, p - 1], Sin[:, :, p - 1], out=buf.S)
        Sin[:, :, p].copy_(buf.S).add_(Sz[:, :, p - 1])
    torch.matmul(M[:, :, P - 1], Sin[:, :, P - 1], out=buf.S)
    buf.S.add_(Sz[:, :, P - 1])
    if timer:
        timer("scan")
    # 4. fix-up of the outputs: o += (M_t^T q_t)^T S_in, one product per segment
    oB = buf.oB.view(B, H, P, Tp, dk)
    o0 = buf.o0.view(B, H, P, Tp, dv)
    o0.add_(torch.matmul(oB, Sin.to(q.dtype)))
    if timer:
        timer("fixup")
    return buf.o0.view(B, H, T, dv), buf.S
