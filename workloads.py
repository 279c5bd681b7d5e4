"""Seeded synthetic inputs for the linear-attention / delta-rule hot path.

This module only draws random inputs; it holds none of the method's
arithmetic.  Both the oracle side (tests, CPU baseline) and the HIP side
(tests, bench) take their inputs from here, so both see the same rounded
values.

Recipe (one ``torch.Generator('cpu')`` seeded with ``1234 + workload index``;
draws happen in this order: q, k, v, beta-logits, gate-logits, initial state;
every draw is float32 and post-processed in float32, then cast to the device
dtype with round-to-nearest-even):

* linear attention: q, k, v ~ N(0, 1).
* delta rule: q, k ~ N(0, 1), each L2-normalised over the head dimension per
  (batch, head, token); q further scaled by 1/sqrt(d_k); v ~ N(0, 1);
  beta = sigmoid(N(0, 1)) per (batch, head, token).
* gated delta rule: as the delta rule, plus gate logits x ~ N(0, 1) per
  (batch, head, token, key channel); the decay is a = exp(-softplus(x)/16) and
  the kernel receives its logarithm g = -softplus(x)/16.  With one decay per
  token (Gated DeltaNet) the logits are drawn per (batch, head, token).
* gated linear attention: q, k, v as the delta rule (no beta), plus one gate
  logit per (batch, head, token) turned into g = -softplus(x)/16 as above.
* decode: state S0 = 0.02 * N(0, 1) (float32), plus a ring of 16 one-token
  inputs drawn as for the delta rule; step i uses ring slot i mod 16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch
import torch.nn.functional as F

BASE_SEED = 1234


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    kind: str          # "la" | "delta" | "gated" | "decode"
    B: int
    H: int
    T: int
    dk: int
    dv: int
    dtype: torch.dtype


# The five workloads of the hot path.  index 0..4.
WORKLOADS = [
    Workload(0, "la_fp32_B1_H2_T64_d16", "la", 1, 2, 64, 16, 16, torch.float32),
    Workload(1, "la_bf16_B8_H12_T1024_d64", "la", 8, 12, 1024, 64, 64, torch.bfloat16),
    Workload(2, "deltanet_bf16_B4_H16_T4096_d128", "delta", 4, 16, 4096, 128, 128,
             torch.bfloat16),
    Workload(3, "gated_deltanet_bf16_B1_H32_T32768_d128", "gated", 1, 32, 32768, 128,
             128, torch.bfloat16),
    # decode: B = sequences, T = timed steps (ring of 16 token inputs)
    Workload(4, "deltanet_decode_N256_H32_d128", "decode", 256, 32, 1000, 128, 128,
             torch.bfloat16),
]
DECODE_RING = 16


def generator(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _normal(gen, shape):
    return torch.randn(*shape, generator=gen, dtype=torch.float32)


def make_la(B, H, T, dk, dv, dtype, seed, init_state=False):
    """q, k, v ~ N(0,1) [B,H,T,d]; optional S0 ~ N(0,1)*0.1 and z0 ~ |N(0,1)|
    (positive, as a running sum of positive features must be)."""
    gen = generator(seed)
    q = _normal(gen, (B, H, T, dk))
    k = _normal(gen, (B, H, T, dk))
    v = _normal(gen, (B, H, T, dv))
    out = dict(q=q.to(dtype), k=k.to(dtype), v=v.to(dtype))
    if init_state:
        out["S0"] = 0.1 * _normal(gen, (B, H, dk, dv))
        out["z0"] = _normal(gen, (B, H, dk)).abs() + 0.5
    return out


def make_delta(B, H, T, dk, dv, dtype, seed, gated=False, init_state=False,
               state_std=0.02):
    """Delta-rule inputs per the recipe above.  g is the log-decay: per key
    channel [B,H,T,dk] with gated=True, per token [B,H,T] with gated="token"."""
    gen = generator(seed)
    q = F.normalize(_normal(gen, (B, H, T, dk)), dim=-1) / math.sqrt(dk)
    k = F.normalize(_normal(gen, (B, H, T, dk)), dim=-1)
    v = _normal(gen, (B, H, T, dv))
    beta = torch.sigmoid(_normal(gen, (B, H, T)))
    out = dict(q=q.to(dtype), k=k.to(dtype), v=v.to(dtype), beta=beta.to(dtype))
    if gated:
        x = _normal(gen, (B, H, T) if gated == "token" else (B, H, T, dk))
        out["g"] = (-F.softplus(x) / 16.0).to(dtype)
    if init_state:
        out["S0"] = state_std * _normal(gen, (B, H, dk, dv))
    return out


def make_gla(B, H, T, dk, dv, dtype, seed, init_state=False, state_std=0.5):
    """Gated linear attention inputs: q, k, v as for the delta rule and the
    per-token log-decay g [B,H,T] = -softplus(x)/16."""
    gen = generator(seed)
    q = F.normalize(_normal(gen, (B, H, T, dk)), dim=-1) / math.sqrt(dk)
    k = F.normalize(_normal(gen, (B, H, T, dk)), dim=-1)
    v = _normal(gen, (B, H, T, dv))
    x = _normal(gen, (B, H, T))
    out = dict(q=q.to(dtype), k=k.to(dtype), v=v.to(dtype),
               g=(-F.softplus(x) / 16.0).to(dtype))
    if init_state:
        out["S0"] = state_std * _normal(gen, (B, H, dk, dv))
    return out


def make_decode(N, H, dk, dv, dtype, seed, gated=False, ring=DECODE_RING):
    """Decode inputs: ring of one-token inputs q, k [ring,N,H,dk], v
    [ring,N,H,dv], beta [ring,N,H] (and g [ring,N,H,dk]); then S0 [N,H,dk,dv]
    float32 = 0.02 * N(0,1)."""
    gen = generator(seed)
    q = F.normalize(_normal(gen, (ring, N, H, dk)), dim=-1) / math.sqrt(dk)
    k = F.normalize(_normal(gen, (ring, N, H, dk)), dim=-1)
    v = _normal(gen, (ring, N, H, dv))
    beta = torch.sigmoid(_normal(gen, (ring, N, H)))
    out = dict(q=q.to(dtype), k=k.to(dtype), v=v.to(dtype), beta=beta.to(dtype))
    if gated:
        x = _normal(gen, (ring, N, H) if gated == "token" else (ring, N, H, dk))
        out["g"] = (-F.softplus(x) / 16.0).to(dtype)
    out["S0"] = 0.02 * _normal(gen, (N, H, dk, dv))
    return out


def make_la_decode(N, H, dk, dv, dtype, seed, ring=DECODE_RING):
    """Linear-attention decode inputs: a ring of one-token q, k, v ~ N(0,1),
    then S0 = 0.02 N(0,1) and z0 = 1 + |N(0,1)| (a normaliser carried from
    earlier tokens is a sum of positive features, so it is kept positive)."""
    gen = generator(seed)
    q = _normal(gen, (ring, N, H, dk))
    k = _normal(gen, (ring, N, H, dk))
    v = _normal(gen, (ring, N, H, dv))
    out = dict(q=q.to(dtype), k=k.to(dtype), v=v.to(dtype))
    out["S0"] = 0.02 * _normal(gen, (N, H, dk, dv))
    out["z0"] = 1.0 + _normal(gen, (N, H, dk)).abs()
    return out


def make_workload(w: Workload):
    seed = BASE_SEED + w.index
    if w.kind == "la":
        return make_la(w.B, w.H, w.T, w.dk, w.dv, w.dtype, seed)
    if w.kind in ("delta", "gated"):
        return make_delta(w.B, w.H, w.T, w.dk, w.dv, w.dtype, seed,
                          gated=(w.kind == "gated"))
    if w.kind == "decode":
        return make_decode(w.B, w.H, w.dk, w.dv, w.dtype, seed)
    raise ValueError(w.kind)
