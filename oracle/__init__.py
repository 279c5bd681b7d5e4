"""CPU float64 oracle for causal linear attention with a fixed d_k x d_v state.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  The HIP library never loads it, and it shares no code with the HIP
library: the arithmetic lives in ``oracle.c`` (plain C, float64, one token at a
time), built into ``liboracle.so`` beside this file.

Functions (both follow the article "From GPT-2 to Kimi K3, explained"):

``la_recurrent``     section "Linear Attention": ELU+1 feature map, running
                     state S and normaliser z, o_t = phi(q_t) S_t / phi(q_t).z_t.
``delta_recurrent``  section "DeltaNet (Parallelizing Linear Transformers with
                     Delta Rule)", sequential prefill loop; with ``g`` given,
                     the decay of sections "Gated Delta Net" (one scalar per
                     token, g [B,H,T]) and "KDA / Kimi Linear" (per key
                     channel, g [B,H,T,dk]) applied to S before each read.
``gla_recurrent``    section "Gated Delta Net", the additive cache with a
                     forgetting factor: S <- a_t S + k_t^T v_t, o_t = q_t S.
``delta_backward``   reverse-mode gradient of the delta rule, ungated or with
                     either gate, token by token: dq, dk, dv, dbeta, dS0
                     (and dg) for the loss sum do . o + sum dS_T * S_T.
``qk_prologue``      section "DeltaNet (Fast Weight Programmers)", the layer's
                     q, k = normalize(silu(.)) (and an optional scale).
``beta_sigmoid``     the same layer's beta = sigmoid(logits), broadcast over
                     heads when the logits have one head.

Inputs may be torch CPU tensors (float32, bfloat16, float64) or numpy arrays
(float32, float64); all inputs of one call share a dtype.  They are read in
their stored precision and widened to float64 inside the C code, so the oracle
sees exactly the rounded values the GPU sees.  Results are numpy float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_F32, _BF16, _F64 = 0, 1, 2


def build(out_path: str = _LIB_PATH, src: str = _SRC, extra_flags=()) -> str:
    """Compile oracle.c with gcc into a shared library.  -O3 with the x86-64-v3
    instruction set (AVX2), not -march=native: the library is built on one
    host and may run on another whose CPU differs.  -ffp-contract=off keeps
    every multiply and add rounded as written (no fused multiply-adds), and
    without -ffast-math the compiler may not reorder floating-point sums, so
    the results are those of the code as written."""
    cmd = ["gcc", "-O3", "-march=x86-64-v3", "-ffp-contract=off", "-std=c11", "-fopenmp",
           "-fPIC", "-shared", *extra_flags, src, "-o", out_path, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


def _bind(lib):
    d = ctypes.c_void_p
    i = ctypes.c_int
    lib.orc_la_recurrent.argtypes = [i, i, i, i, i, d, d, d, i, d, d, d, d, d, i]
    lib.orc_la_recurrent.restype = i
    lib.orc_delta_recurrent.argtypes = [i, i, i, i, i, d, d, d, d, d, i, i, d, d, d, i]
    lib.orc_delta_recurrent.restype = i
    lib.orc_gla_recurrent.argtypes = [i, i, i, i, i, d, d, d, d, i, d, d, d, i]
    lib.orc_gla_recurrent.restype = i
    lib.orc_delta_backward.argtypes = [i, i, i, i, i, d, d, d, d, d, i, i, d, d, d,
                                       d, d, d, d, d, d, i]
    lib.orc_delta_backward.restype = i
    lib.orc_qk_prologue.argtypes = [ctypes.c_long, i, d, i, i, ctypes.c_double, d]
    lib.orc_qk_prologue.restype = i
    lib.orc_beta_sigmoid.argtypes = [i, i, i, i, d, i, d]
    lib.orc_beta_sigmoid.restype = i
    lib.orc_max_threads.argtypes = []
    lib.orc_max_threads.restype = i
    return lib


def load(path: str | None = None):
    """Load liboracle.so (building it first if it is absent).  With ``path``
    given, load that library instead (used to test planted mistakes)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def max_threads() -> int:
    return int(load().orc_max_threads())


def _as_buffer(x):
    """Return (keepalive, pointer, dtype-code) for a CPU tensor or array,
    without changing its stored precision."""
    try:
        import torch
    except ImportError:  # pragma: no cover
        torch = None
    if torch is not None and isinstance(x, torch.Tensor):
        if x.device.type != "cpu":
            raise ValueError("oracle inputs must be CPU tensors")
        x = x.contiguous()
        if x.dtype == torch.bfloat16:
            return x, x.data_ptr(), _BF16
        if x.dtype == torch.float32:
            return x, x.data_ptr(), _F32
        if x.dtype == torch.float64:
            return x, x.data_ptr(), _F64
        raise ValueError(f"unsupported dtype {x.dtype}")
    a = np.ascontiguousarray(x)
    if a.dtype == np.float32:
        return a, a.ctypes.data, _F32
    if a.dtype == np.float64:
        return a, a.ctypes.data, _F64
    raise ValueError(f"unsupported dtype {a.dtype}")


def _state64(x, shape):
    if x is None:
        return None, None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().double().numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64)).reshape(shape)
    return a, a.ctypes.data


def la_recurrent(q, k, v, S0=None, z0=None, nthreads: int = 0, lib=None):
    """ELU+1 linear attention with normaliser, token by token.
    q, k [B,H,T,dk]; v [B,H,T,dv]; S0 [B,H,dk,dv] and z0 [B,H,dk] optional
    (float64-convertible).  Returns (o [B,H,T,dv], S [B,H,dk,dv], z [B,H,dk])."""
    lib = lib or load()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    bufs = [_as_buffer(t) for t in (q, k, v)]
    dts = {b[2] for b in bufs}
    if len(dts) != 1:
        raise ValueError("q, k, v must share a dtype")
    s0, s0p = _state64(S0, (B, H, dk, dv))
    z0a, z0p = _state64(z0, (B, H, dk))
    o = np.empty((B, H, T, dv), np.float64)
    S = np.empty((B, H, dk, dv), np.float64)
    z = np.empty((B, H, dk), np.float64)
    rc = lib.orc_la_recurrent(B, H, T, dk, dv, bufs[0][1], bufs[1][1], bufs[2][1],
                              dts.pop(), s0p, z0p, o.ctypes.data, S.ctypes.data,
                              z.ctypes.data, int(nthreads))
    if rc != 0:
        raise MemoryError("oracle allocation failed")
    return o, S, z


def delta_recurrent(q, k, v, beta, g=None, S0=None, nthreads: int = 0, lib=None,
                    want_o: bool = True):
    """Delta rule (g None) or gated delta rule, token by token.
    q, k [B,H,T,dk]; v [B,H,T,dv]; beta [B,H,T]; g log-decay, [B,H,T,dk] per
    key channel or [B,H,T] per token, or None; S0 [B,H,dk,dv] or None.
    Returns (o [B,H,T,dv] or None, S [B,H,dk,dv])."""
    lib = lib or load()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    tensors = [q, k, v, beta] + ([g] if g is not None else [])
    bufs = [_as_buffer(t) for t in tensors]
    dts = {b[2] for b in bufs}
    if len(dts) != 1:
        raise ValueError("q, k, v, beta (and g) must share a dtype")
    gp = bufs[4][1] if g is not None else None
    per_channel = 1
    if g is not None:
        if tuple(g.shape) == (B, H, T):
            per_channel = 0
        elif tuple(g.shape) != (B, H, T, dk):
            raise ValueError(f"g must be [B,H,T] or [B,H,T,dk], got {tuple(g.shape)}")
    s0, s0p = _state64(S0, (B, H, dk, dv))
    o = np.empty((B, H, T, dv), np.float64) if want_o else None
    S = np.empty((B, H, dk, dv), np.float64)
    rc = lib.orc_delta_recurrent(B, H, T, dk, dv, bufs[0][1], bufs[1][1], bufs[2][1],
                                 bufs[3][1], gp, per_channel, dts.pop(), s0p,
                                 o.ctypes.data if want_o else None, S.ctypes.data,
                                 int(nthreads))
    if rc != 0:
        raise MemoryError("oracle allocation failed")
    return o, S


def gla_recurrent(q, k, v, g=None, S0=None, nthreads: int = 0, lib=None):
    """Gated linear attention without a normaliser, token by token:
    S <- exp(g_t) S + k_t^T v_t, o_t = q_t S.  q, k [B,H,T,dk]; v [B,H,T,dv];
    g [B,H,T] log-decay or None; S0 [B,H,dk,dv] or None.
    Returns (o [B,H,T,dv], S [B,H,dk,dv])."""
    lib = lib or load()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    tensors = [q, k, v] + ([g] if g is not None else [])
    bufs = [_as_buffer(t) for t in tensors]
    dts = {b[2] for b in bufs}
    if len(dts) != 1:
        raise ValueError("q, k, v (and g) must share a dtype")
    if g is not None and tuple(g.shape) != (B, H, T):
        raise ValueError(f"g must be [B,H,T], got {tuple(g.shape)}")
    gp = bufs[3][1] if g is not None else None
    s0, s0p = _state64(S0, (B, H, dk, dv))
    o = np.empty((B, H, T, dv), np.float64)
    S = np.empty((B, H, dk, dv), np.float64)
    rc = lib.orc_gla_recurrent(B, H, T, dk, dv, bufs[0][1], bufs[1][1], bufs[2][1], gp,
                               dts.pop(), s0p, o.ctypes.data, S.ctypes.data, int(nthreads))
    if rc != 0:
        raise MemoryError("oracle allocation failed")
    return o, S


def delta_backward(q, k, v, beta, dO, S0=None, dST=None, g=None, nthreads: int = 0,
                   lib=None):
    """Gradients of the delta rule (g None) or the gated delta rule for the
    loss sum(dO * o) + sum(dST * S_T).  q, k [B,H,T,dk]; v, dO [B,H,T,dv];
    beta [B,H,T]; g log-decay, [B,H,T] per token or [B,H,T,dk] per key
    channel (one dtype with the others); S0 and dST [B,H,dk,dv] or None.
    Returns (dq, dk, dv, dbeta, dS0) as float64, and dg (g's shape) after
    them when g is given."""
    lib = lib or load()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    tensors = [q, k, v, beta, dO] + ([g] if g is not None else [])
    bufs = [_as_buffer(t) for t in tensors]
    dts = {b[2] for b in bufs}
    if len(dts) != 1:
        raise ValueError("q, k, v, beta, dO (and g) must share a dtype")
    per_channel = 0
    if g is not None:
        if tuple(g.shape) == (B, H, T, dk):
            per_channel = 1
        elif tuple(g.shape) != (B, H, T):
            raise ValueError(f"g must be [B,H,T] or [B,H,T,dk], got {tuple(g.shape)}")
    s0, s0p = _state64(S0, (B, H, dk, dv))
    dst, dstp = _state64(dST, (B, H, dk, dv))
    dq = np.empty((B, H, T, dk), np.float64)
    dkk = np.empty((B, H, T, dk), np.float64)
    dvv = np.empty((B, H, T, dv), np.float64)
    db = np.empty((B, H, T), np.float64)
    dS0 = np.empty((B, H, dk, dv), np.float64)
    dg = np.empty(tuple(g.shape), np.float64) if g is not None else None
    rc = lib.orc_delta_backward(B, H, T, dk, dv, bufs[0][1], bufs[1][1], bufs[2][1],
                                bufs[3][1], bufs[5][1] if g is not None else None,
                                per_channel, dts.pop(), s0p, bufs[4][1], dstp,
                                dq.ctypes.data, dkk.ctypes.data, dvv.ctypes.data,
                                db.ctypes.data, dS0.ctypes.data,
                                dg.ctypes.data if g is not None else None, int(nthreads))
    if rc != 0:
        raise MemoryError("oracle allocation failed")
    if g is None:
        return dq, dkk, dvv, db, dS0
    return dq, dkk, dvv, db, dS0, dg


def qk_prologue(x, apply_silu: bool = True, scale: float = 1.0, lib=None):
    """scale * L2-normalise(silu(x)) over the last dimension (silu skipped
    when apply_silu is False).  x [..., d]; returns float64 of x's shape."""
    lib = lib or load()
    buf = _as_buffer(x)
    d = x.shape[-1]
    rows = int(np.prod(x.shape[:-1]))
    out = np.empty(tuple(x.shape), np.float64)
    lib.orc_qk_prologue(rows, d, buf[1], buf[2], int(bool(apply_silu)), float(scale),
                        out.ctypes.data)
    return out


def beta_sigmoid(logits, H: int, lib=None):
    """sigmoid(logits) for logits [B, Hb, T] with Hb = 1 (shared by all H
    heads) or Hb = H; returns float64 [B, H, T]."""
    lib = lib or load()
    buf = _as_buffer(logits)
    B, Hb, T = logits.shape
    out = np.empty((B, H, T), np.float64)
    lib.orc_beta_sigmoid(B, Hb, H, T, buf[1], buf[2], out.ctypes.data)
    return out
