"""Causal linear attention with a fixed d_k x d_v state on AMD MI355X (gfx950).

A thin ctypes binding over ``liblinattn.so``, the HIP library whose C ABI is
declared in ``include/linattn.h``.  The functions below carry the same names
as the C entry points and only marshal arguments: check devices, dtypes,
shapes and contiguity, allocate outputs the caller did not pass, and hand raw
device pointers plus the current HIP stream to the library.  Every step of
the computation runs in the library's kernels; there is no fallback.

Build the library with ``python -m delta_rule_recurrent_chunkwise_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "la_prefill", "la_decode_step", "deltanet_prefill", "deltanet_decode_step",
    "gated_deltanet_prefill", "gated_deltanet_decode_step", "gla_prefill",
    "gla_decode_step", "deltanet_prefill_backward", "gated_deltanet_prefill_backward",
    "kda_prefill_backward", "deltanet_prologue", "deltanet_prefill_segmented",
    "deltanet_prefill_segments", "deltanet_prefill_segmented_workspace_bytes", "la_strerror",
    "la_prefill_workspace_bytes", "deltanet_prefill_workspace_bytes",
    "gla_prefill_workspace_bytes", "deltanet_prefill_backward_workspace_bytes",
    "gated_deltanet_prefill_backward_workspace_bytes", "kda_prefill_backward_workspace_bytes",
    "la_prefill_noalloc",
    "library", "LIB_PATH",
    "EXPORTED_SYMBOLS",
    "LinAttnError",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblinattn.so")
COMPUTE_ENTRIES = ("la_prefill", "la_decode_step", "deltanet_prefill",
                   "deltanet_decode_step", "gated_deltanet_prefill",
                   "gated_deltanet_decode_step", "gla_prefill", "gla_decode_step",
                   "deltanet_prefill_backward", "gated_deltanet_prefill_backward",
                   "kda_prefill_backward", "deltanet_prologue", "deltanet_prefill_segmented")
WORKSPACE_QUERIES = ("la_prefill_workspace_bytes", "deltanet_prefill_workspace_bytes",
                     "gla_prefill_workspace_bytes",
                     "deltanet_prefill_backward_workspace_bytes",
                     "gated_deltanet_prefill_backward_workspace_bytes",
                     "kda_prefill_backward_workspace_bytes",
                     "deltanet_prefill_segmented_workspace_bytes")
EXPORTED_SYMBOLS = COMPUTE_ENTRIES + WORKSPACE_QUERIES + ("deltanet_prefill_segments",
                                                          "la_prefill_noalloc", "la_strerror")
NOALLOC_SCRATCH_BYTES = 64 << 20

LA_DTYPE_F32, LA_DTYPE_BF16 = 0, 1
_DTYPES = {torch.float32: LA_DTYPE_F32, torch.bfloat16: LA_DTYPE_BF16}

_lib = None


class LinAttnError(RuntimeError):
    """A negative return code from liblinattn.so."""

    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn}: {msg} (code {code})")
        self.code = code


def library():
    """Load liblinattn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m delta_rule_recurrent_chunkwise_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        lib.la_prefill.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, P, Z, P]
        lib.la_decode_step.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P]
        lib.deltanet_prefill.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, Z, P]
        lib.deltanet_decode_step.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, P]
        lib.gated_deltanet_prefill.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, P]
        lib.gated_deltanet_decode_step.argtypes = lib.deltanet_decode_step.argtypes
        lib.gla_prefill.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, P, Z, P]
        lib.gla_decode_step.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P]
        lib.deltanet_prefill_backward.argtypes = [P] * 12 + [I] * 6 + [P, Z, P]
        lib.gated_deltanet_prefill_backward.argtypes = [P] * 14 + [I] * 6 + [P, Z, P]
        lib.kda_prefill_backward.argtypes = [P] * 14 + [I] * 6 + [P, Z, P]
        lib.deltanet_prologue.argtypes = [P] * 6 + [I] * 6 + [ctypes.c_float, I, P]
        lib.deltanet_prefill_segmented.argtypes = [P] * 5 + [I, P, P] + [I] * 8 + [P, Z, P]
        for fn in COMPUTE_ENTRIES:
            getattr(lib, fn).restype = I
        lib.la_prefill_workspace_bytes.argtypes = [I] * 6
        lib.deltanet_prefill_workspace_bytes.argtypes = [I] * 7
        lib.gla_prefill_workspace_bytes.argtypes = [I] * 6
        lib.deltanet_prefill_backward_workspace_bytes.argtypes = [I] * 6
        lib.gated_deltanet_prefill_backward_workspace_bytes.argtypes = [I] * 6
        lib.kda_prefill_backward_workspace_bytes.argtypes = [I] * 6
        lib.deltanet_prefill_segmented_workspace_bytes.argtypes = [I] * 8
        lib.deltanet_prefill_segments.argtypes = [I] * 5
        lib.deltanet_prefill_segments.restype = I
        for fn in WORKSPACE_QUERIES:
            getattr(lib, fn).restype = Z
        lib.la_prefill_noalloc.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, P]
        lib.la_prefill_noalloc.restype = I
        lib.la_strerror.argtypes = [I]
        lib.la_strerror.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def la_strerror(code: int) -> str:
    return library().la_strerror(int(code)).decode()


def _dt(dtype) -> int:
    return dtype if isinstance(dtype, int) else _DTYPES[dtype]


def la_prefill_workspace_bytes(B, H, T, dk, dv, dtype) -> int:
    """Bytes of workspace la_prefill needs for these sizes (0: none)."""
    return int(library().la_prefill_workspace_bytes(B, H, T, dk, dv, _dt(dtype)))


def deltanet_prefill_workspace_bytes(gated, B, H, T, dk, dv, dtype) -> int:
    """Bytes of workspace deltanet_prefill needs (gated: g given; 0: none)."""
    return int(library().deltanet_prefill_workspace_bytes(int(bool(gated)), B, H, T, dk, dv,
                                                          _dt(dtype)))


def gla_prefill_workspace_bytes(B, H, T, dk, dv, dtype) -> int:
    """Bytes of workspace gla_prefill needs for these sizes (0: none)."""
    return int(library().gla_prefill_workspace_bytes(B, H, T, dk, dv, _dt(dtype)))


def deltanet_prefill_backward_workspace_bytes(B, H, T, dk, dv, dtype) -> int:
    """Bytes of workspace deltanet_prefill_backward needs."""
    return int(library().deltanet_prefill_backward_workspace_bytes(B, H, T, dk, dv, _dt(dtype)))


def gated_deltanet_prefill_backward_workspace_bytes(B, H, T, dk, dv, dtype) -> int:
    """Bytes of workspace gated_deltanet_prefill_backward needs."""
    return int(library().gated_deltanet_prefill_backward_workspace_bytes(B, H, T, dk, dv,
                                                                         _dt(dtype)))


def kda_prefill_backward_workspace_bytes(B, H, T, dk, dv, dtype) -> int:
    """Bytes of workspace kda_prefill_backward needs."""
    return int(library().kda_prefill_backward_workspace_bytes(B, H, T, dk, dv, _dt(dtype)))


def _check(fn: str, rc: int):
    if rc != 0:
        raise LinAttnError(fn, rc, la_strerror(rc))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _inputs(fn, tensors, shapes):
    """All given tensors on one GPU, contiguous, one dtype in _DTYPES, with the
    expected shapes."""
    dev = None
    dtype = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{fn}: {name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{fn}: {name} must be contiguous")
        if dev is None:
            dev, dtype = t.device, t.dtype
        if t.device != dev:
            raise ValueError(f"{fn}: all tensors must be on one device")
        if t.dtype != dtype:
            raise ValueError(f"{fn}: {name} has dtype {t.dtype}, expected {dtype}")
        if tuple(t.shape) != tuple(shapes[name]):
            raise ValueError(f"{fn}: {name} has shape {tuple(t.shape)}, "
                             f"expected {tuple(shapes[name])}")
    if dtype not in _DTYPES:
        raise ValueError(f"{fn}: dtype must be float32 or bfloat16, got {dtype}")
    return dev, dtype


def _state(fn, name, t, shape, dev):
    if t is None:
        return torch.empty(shape, device=dev, dtype=torch.float32)
    if (not t.is_cuda or t.device != dev or t.dtype != torch.float32
            or not t.is_contiguous() or tuple(t.shape) != tuple(shape)):
        raise ValueError(f"{fn}: {name} must be a contiguous float32 tensor of shape "
                         f"{tuple(shape)} on {dev}")
    return t


def _workspace(nbytes, dev, workspace):
    """(pointer, size) of a workspace of at least nbytes bytes: the caller's
    uint8 tensor if given, else a fresh torch allocation (256-byte aligned)
    that lives until the call returns; the library's kernels are enqueued on
    the current stream, so torch's caching allocator reuses the block only
    for work ordered after them."""
    if nbytes == 0:
        return None, 0, None
    if workspace is None:
        workspace = torch.empty(int(nbytes), device=dev, dtype=torch.uint8)
    elif (not isinstance(workspace, torch.Tensor) or workspace.device != dev
          or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(), workspace


def _out(fn, o, shape, dev, dtype):
    if o is None:
        return torch.empty(shape, device=dev, dtype=dtype)
    if (not o.is_cuda or o.device != dev or o.dtype != dtype or not o.is_contiguous()
            or tuple(o.shape) != tuple(shape)):
        raise ValueError(f"{fn}: o must be a contiguous {dtype} tensor of shape {tuple(shape)}")
    return o


def la_prefill(q, k, v, S=None, z=None, use_initial_state=False, o=None, stream=None,
               workspace=None):
    """ELU+1 linear attention with normaliser over q, k [B,H,T,dk], v [B,H,T,dv].
    Returns (o [B,H,T,dv], S [B,H,dk,dv] fp32, z [B,H,dk] fp32).  With
    use_initial_state the given S, z are the initial state; they are
    overwritten with the final state.  workspace: an optional device tensor
    of at least la_prefill_workspace_bytes(...) bytes (allocated here if
    None and one is needed)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev, dtype = _inputs("la_prefill", dict(q=q, k=k, v=v),
                         dict(q=(B, H, T, dk), k=(B, H, T, dk), v=(B, H, T, dv)))
    if use_initial_state and (S is None or z is None):
        raise ValueError("la_prefill: use_initial_state needs S and z")
    S = _state("la_prefill", "S", S, (B, H, dk, dv), dev)
    z = _state("la_prefill", "z", z, (B, H, dk), dev)
    o = _out("la_prefill", o, (B, H, T, dv), dev, dtype)
    wp, wn, _keep = _workspace(la_prefill_workspace_bytes(B, H, T, dk, dv, dtype), dev, workspace)
    rc = library().la_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(S), _ptr(z),
                              int(bool(use_initial_state)), B, H, T, dk, dv,
                              _DTYPES[dtype], wp, wn, _stream(dev, stream))
    _check("la_prefill", rc)
    return o, S, z


def la_prefill_noalloc(q, k, v, o, S, z, use_initial_state=False, stream=None):
    """la_prefill for callers that cannot allocate: o [B,H,T,dv], S [B,H,dk,dv]
    and z [B,H,dk] (fp32) must be given, and nothing is allocated here or in
    the library (its scratch is a fixed 64 MiB array per GPU).  Raises
    LinAttnError (LA_ERR_SCRATCH_LIMIT) if the sizes need more scratch than
    that.  Calls that may overlap on one GPU must not be made."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev, dtype = _inputs("la_prefill_noalloc", dict(q=q, k=k, v=v, o=o),
                         dict(q=(B, H, T, dk), k=(B, H, T, dk), v=(B, H, T, dv),
                              o=(B, H, T, dv)))
    if S is None or z is None:
        raise ValueError("la_prefill_noalloc: S and z must be given")
    _state("la_prefill_noalloc", "S", S, (B, H, dk, dv), dev)
    _state("la_prefill_noalloc", "z", z, (B, H, dk), dev)
    rc = library().la_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(S), _ptr(z),
                                      int(bool(use_initial_state)), B, H, T, dk, dv,
                                      _DTYPES[dtype], _stream(dev, stream))
    _check("la_prefill_noalloc", rc)
    return o, S, z


def la_decode_step(q, k, v, S, z, o=None, stream=None):
    """One token per sequence: q, k [N,H,dk], v [N,H,dv]; S [N,H,dk,dv] and
    z [N,H,dk] (fp32) updated in place.  Returns o [N,H,dv]."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev, dtype = _inputs("la_decode_step", dict(q=q, k=k, v=v),
                         dict(q=(N, H, dk), k=(N, H, dk), v=(N, H, dv)))
    S = _state("la_decode_step", "S", S, (N, H, dk, dv), dev)
    z = _state("la_decode_step", "z", z, (N, H, dk), dev)
    o = _out("la_decode_step", o, (N, H, dv), dev, dtype)
    rc = library().la_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(S), _ptr(z),
                                  N, H, dk, dv, _DTYPES[dtype], _stream(dev, stream))
    _check("la_decode_step", rc)
    return o


def deltanet_prefill(q, k, v, beta, g=None, S=None, use_initial_state=False, o=None,
                     stream=None, workspace=None):
    """Delta rule (g None) or per-key-channel gated delta rule (g = log-decay
    [B,H,T,dk]) over q, k [B,H,T,dk], v [B,H,T,dv], beta [B,H,T].
    Returns (o [B,H,T,dv], S [B,H,dk,dv] fp32)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev, dtype = _inputs("deltanet_prefill", dict(q=q, k=k, v=v, beta=beta, g=g),
                         dict(q=(B, H, T, dk), k=(B, H, T, dk), v=(B, H, T, dv),
                              beta=(B, H, T), g=(B, H, T, dk)))
    if use_initial_state and S is None:
        raise ValueError("deltanet_prefill: use_initial_state needs S")
    S = _state("deltanet_prefill", "S", S, (B, H, dk, dv), dev)
    o = _out("deltanet_prefill", o, (B, H, T, dv), dev, dtype)
    wp, wn, _keep = _workspace(deltanet_prefill_workspace_bytes(g is not None, B, H, T, dk, dv, dtype),
                               dev, workspace)
    rc = library().deltanet_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                    _ptr(o), _ptr(S), int(bool(use_initial_state)),
                                    B, H, T, dk, dv, _DTYPES[dtype], wp, wn,
                                    _stream(dev, stream))
    _check("deltanet_prefill", rc)
    return o, S


def deltanet_decode_step(q, k, v, beta, S, g=None, o=None, stream=None):
    """One token per sequence: q, k [N,H,dk], v [N,H,dv], beta [N,H],
    g [N,H,dk] or None; S [N,H,dk,dv] fp32 updated in place.  Returns o."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev, dtype = _inputs("deltanet_decode_step", dict(q=q, k=k, v=v, beta=beta, g=g),
                         dict(q=(N, H, dk), k=(N, H, dk), v=(N, H, dv), beta=(N, H),
                              g=(N, H, dk)))
    S = _state("deltanet_decode_step", "S", S, (N, H, dk, dv), dev)
    o = _out("deltanet_decode_step", o, (N, H, dv), dev, dtype)
    rc = library().deltanet_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                        _ptr(o), _ptr(S), N, H, dk, dv, _DTYPES[dtype],
                                        _stream(dev, stream))
    _check("deltanet_decode_step", rc)
    return o


def gated_deltanet_prefill(q, k, v, beta, g, S=None, use_initial_state=False, o=None,
                           stream=None):
    """Delta rule with one decay per token (g = log-decay [B,H,T]) over
    q, k [B,H,T,dk], v [B,H,T,dv], beta [B,H,T].
    Returns (o [B,H,T,dv], S [B,H,dk,dv] fp32)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if g is None:
        raise ValueError("gated_deltanet_prefill: g is required")
    dev, dtype = _inputs("gated_deltanet_prefill", dict(q=q, k=k, v=v, beta=beta, g=g),
                         dict(q=(B, H, T, dk), k=(B, H, T, dk), v=(B, H, T, dv),
                              beta=(B, H, T), g=(B, H, T)))
    if use_initial_state and S is None:
        raise ValueError("gated_deltanet_prefill: use_initial_state needs S")
    S = _state("gated_deltanet_prefill", "S", S, (B, H, dk, dv), dev)
    o = _out("gated_deltanet_prefill", o, (B, H, T, dv), dev, dtype)
    rc = library().gated_deltanet_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                          _ptr(o), _ptr(S), int(bool(use_initial_state)),
                                          B, H, T, dk, dv, _DTYPES[dtype],
                                          _stream(dev, stream))
    _check("gated_deltanet_prefill", rc)
    return o, S


_SEG_GATES = {None: 0, "channel": 1, "token": 2}


def deltanet_prefill_segments(B, H, T, dk, dv) -> int:
    """The segment count deltanet_prefill_segmented picks for segments=0
    (1: one pass over the whole sequence; 0: invalid sizes)."""
    return int(library().deltanet_prefill_segments(B, H, T, dk, dv))


def deltanet_prefill_segmented_workspace_bytes(gate, B, H, T, dk, dv, dtype, segments=0) -> int:
    """Bytes of workspace deltanet_prefill_segmented needs; gate is None,
    "channel" (g [B,H,T,dk]) or "token" (g [B,H,T])."""
    return int(library().deltanet_prefill_segmented_workspace_bytes(
        _SEG_GATES[gate], B, H, T, dk, dv, _dt(dtype), int(segments)))


def deltanet_prefill_segmented(q, k, v, beta, g=None, gate=None, S=None, use_initial_state=False,
                               segments=0, o=None, stream=None, workspace=None):
    """The delta rule of deltanet_prefill (gate None or "channel": g [B,H,T,dk])
    or gated_deltanet_prefill (gate "token": g [B,H,T]) with each head's
    sequence processed as `segments` segments side by side (0: the library
    chooses; 1: one pass).  q, k [B,H,T,dk], v [B,H,T,dv], beta [B,H,T], bf16.
    Returns (o [B,H,T,dv], S [B,H,dk,dv] fp32)."""
    fn = "deltanet_prefill_segmented"
    if gate not in _SEG_GATES:
        raise ValueError(f"{fn}: gate must be None, 'channel' or 'token'")
    if (g is None) != (gate is None):
        raise ValueError(f"{fn}: g must be given exactly when gate is")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    gshape = (B, H, T, dk) if gate == "channel" else (B, H, T)
    dev, dtype = _inputs(fn, dict(q=q, k=k, v=v, beta=beta, g=g),
                         dict(q=(B, H, T, dk), k=(B, H, T, dk), v=(B, H, T, dv),
                              beta=(B, H, T), g=gshape))
    if use_initial_state and S is None:
        raise ValueError(f"{fn}: use_initial_state needs S")
    S = _state(fn, "S", S, (B, H, dk, dv), dev)
    o = _out(fn, o, (B, H, T, dv), dev, dtype)
    wp, wn, _keep = _workspace(
        deltanet_prefill_segmented_workspace_bytes(gate, B, H, T, dk, dv, dtype, segments),
        dev, workspace)
    rc = library().deltanet_prefill_segmented(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                              _SEG_GATES[gate], _ptr(o), _ptr(S),
                                              int(bool(use_initial_state)), B, H, T, dk, dv,
                                              _DTYPES[dtype], int(segments), wp, wn,
                                              _stream(dev, stream))
    _check(fn, rc)
    return o, S


def gated_deltanet_decode_step(q, k, v, beta, g, S, o=None, stream=None):
    """One token per sequence of gated_deltanet_prefill: q, k [N,H,dk],
    v [N,H,dv], beta [N,H], g [N,H]; S [N,H,dk,dv] fp32 updated in place.
    Returns o [N,H,dv]."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    if g is None:
        raise ValueError("gated_deltanet_decode_step: g is required")
    dev, dtype = _inputs("gated_deltanet_decode_step", dict(q=q, k=k, v=v, beta=beta, g=g),
                         dict(q=(N, H, dk), k=(N, H, dk), v=(N, H, dv), beta=(N, H),
                              g=(N, H)))
    S = _state("gated_deltanet_decode_step", "S", S, (N, H, dk, dv), dev)
    o = _out("gated_deltanet_decode_step", o, (N, H, dv), dev, dtype)
    rc = library().gated_deltanet_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                              _ptr(g), _ptr(o), _ptr(S), N, H, dk, dv,
                                              _DTYPES[dtype], _stream(dev, stream))
    _check("gated_deltanet_decode_step", rc)
    return o


def gla_prefill(q, k, v, g=None, S=None, use_initial_state=False, o=None, stream=None,
                workspace=None):
    """Gated linear attention S <- a S + k^T v, o = q S over q, k [B,H,T,dk],
    v [B,H,T,dv], g = log-decay [B,H,T] or None.
    Returns (o [B,H,T,dv], S [B,H,dk,dv] fp32)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev, dtype = _inputs("gla_prefill", dict(q=q, k=k, v=v, g=g),
                         dict(q=(B, H, T, dk), k=(B, H, T, dk), v=(B, H, T, dv),
                              g=(B, H, T)))
    if use_initial_state and S is None:
        raise ValueError("gla_prefill: use_initial_state needs S")
    S = _state("gla_prefill", "S", S, (B, H, dk, dv), dev)
    o = _out("gla_prefill", o, (B, H, T, dv), dev, dtype)
    wp, wn, _keep = _workspace(gla_prefill_workspace_bytes(B, H, T, dk, dv, dtype), dev, workspace)
    rc = library().gla_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(o), _ptr(S),
                               int(bool(use_initial_state)), B, H, T, dk, dv,
                               _DTYPES[dtype], wp, wn, _stream(dev, stream))
    _check("gla_prefill", rc)
    return o, S


def gla_decode_step(q, k, v, S, g=None, o=None, stream=None):
    """One token per sequence of gla_prefill: q, k [N,H,dk], v [N,H,dv],
    g [N,H] or None; S [N,H,dk,dv] fp32 updated in place.  Returns o."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev, dtype = _inputs("gla_decode_step", dict(q=q, k=k, v=v, g=g),
                         dict(q=(N, H, dk), k=(N, H, dk), v=(N, H, dv), g=(N, H)))
    S = _state("gla_decode_step", "S", S, (N, H, dk, dv), dev)
    o = _out("gla_decode_step", o, (N, H, dv), dev, dtype)
    rc = library().gla_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(o), _ptr(S),
                                   N, H, dk, dv, _DTYPES[dtype], _stream(dev, stream))
    _check("gla_decode_step", rc)
    return o


def deltanet_prefill_backward(q, k, v, beta, dO, S0=None, dST=None, want_dS0=False,
                              stream=None, workspace=None):
    """Gradients of deltanet_prefill (no gate) for the loss
    sum(dO * o) + sum(dST * S_T): returns (dq, dk, dv, dbeta, dS0), dS0 None
    unless want_dS0.  q, k [B,H,T,dk]; v, dO [B,H,T,dv]; beta [B,H,T] (one
    dtype); S0, dST [B,H,dk,dv] fp32 or None."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev, dtype = _inputs("deltanet_prefill_backward", dict(q=q, k=k, v=v, beta=beta, dO=dO),
                         dict(q=(B, H, T, dk), k=(B, H, T, dk), v=(B, H, T, dv),
                              beta=(B, H, T), dO=(B, H, T, dv)))
    for name, t in (("S0", S0), ("dST", dST)):
        if t is not None:
            _state("deltanet_prefill_backward", name, t, (B, H, dk, dv), dev)
    dq = torch.empty_like(q)
    dkk = torch.empty_like(k)
    dvv = torch.empty_like(v)
    db = torch.empty_like(beta)
    dS0 = torch.empty(B, H, dk, dv, device=dev, dtype=torch.float32) if want_dS0 else None
    wp, wn, _keep = _workspace(deltanet_prefill_backward_workspace_bytes(B, H, T, dk, dv, dtype),
                               dev, workspace)
    rc = library().deltanet_prefill_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S0), _ptr(dO), _ptr(dST), _ptr(dq),
        _ptr(dkk), _ptr(dvv), _ptr(db), _ptr(dS0), B, H, T, dk, dv, _DTYPES[dtype],
        wp, wn, _stream(dev, stream))
    _check("deltanet_prefill_backward", rc)
    return dq, dkk, dvv, db, dS0


def gated_deltanet_prefill_backward(q, k, v, beta, g, dO, S0=None, dST=None, want_dS0=False,
                                    stream=None, workspace=None):
    """Gradients of gated_deltanet_prefill (one log-decay per token) for the
    loss sum(dO * o) + sum(dST * S_T): returns (dq, dk, dv, dbeta, dg, dS0),
    dS0 None unless want_dS0.  g [B,H,T] in the inputs' dtype; the rest as
    deltanet_prefill_backward."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev, dtype = _inputs("gated_deltanet_prefill_backward",
                         dict(q=q, k=k, v=v, beta=beta, g=g, dO=dO),
                         dict(q=(B, H, T, dk), k=(B, H, T, dk), v=(B, H, T, dv),
                              beta=(B, H, T), g=(B, H, T), dO=(B, H, T, dv)))
    for name, t in (("S0", S0), ("dST", dST)):
        if t is not None:
            _state("gated_deltanet_prefill_backward", name, t, (B, H, dk, dv), dev)
    dq = torch.empty_like(q)
    dkk = torch.empty_like(k)
    dvv = torch.empty_like(v)
    db = torch.empty_like(beta)
    dg = torch.empty_like(g)
    dS0 = torch.empty(B, H, dk, dv, device=dev, dtype=torch.float32) if want_dS0 else None
    wp, wn, _keep = _workspace(
        gated_deltanet_prefill_backward_workspace_bytes(B, H, T, dk, dv, dtype), dev, workspace)
    rc = library().gated_deltanet_prefill_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0), _ptr(dO), _ptr(dST),
        _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(db), _ptr(dg), _ptr(dS0), B, H, T, dk, dv,
        _DTYPES[dtype], wp, wn, _stream(dev, stream))
    _check("gated_deltanet_prefill_backward", rc)
    return dq, dkk, dvv, db, dg, dS0


def kda_prefill_backward(q, k, v, beta, g, dO, S0=None, dST=None, want_dS0=False,
                         stream=None, workspace=None):
    """Gradients of deltanet_prefill with a per-key-channel gate (g =
    log-decay [B,H,T,dk]) for the loss sum(dO * o) + sum(dST * S_T): returns
    (dq, dk, dv, dbeta, dg, dS0), dS0 None unless want_dS0.  bf16 inputs; the
    rest as deltanet_prefill_backward."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev, dtype = _inputs("kda_prefill_backward", dict(q=q, k=k, v=v, beta=beta, g=g, dO=dO),
                         dict(q=(B, H, T, dk), k=(B, H, T, dk), v=(B, H, T, dv),
                              beta=(B, H, T), g=(B, H, T, dk), dO=(B, H, T, dv)))
    for name, t in (("S0", S0), ("dST", dST)):
        if t is not None:
            _state("kda_prefill_backward", name, t, (B, H, dk, dv), dev)
    dq = torch.empty_like(q)
    dkk = torch.empty_like(k)
    dvv = torch.empty_like(v)
    db = torch.empty_like(beta)
    dg = torch.empty_like(g)
    dS0 = torch.empty(B, H, dk, dv, device=dev, dtype=torch.float32) if want_dS0 else None
    wp, wn, _keep = _workspace(kda_prefill_backward_workspace_bytes(B, H, T, dk, dv, dtype), dev,
                               workspace)
    rc = library().kda_prefill_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0), _ptr(dO), _ptr(dST),
        _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(db), _ptr(dg), _ptr(dS0), B, H, T, dk, dv,
        _DTYPES[dtype], wp, wn, _stream(dev, stream))
    _check("kda_prefill_backward", rc)
    return dq, dkk, dvv, db, dg, dS0


def deltanet_prologue(q, k, beta_logits=None, apply_silu=True, q_scale=1.0, out=None,
                      stream=None):
    """q, k [B,H,T,dk] -> (q_scale * normalize(silu(q)), normalize(silu(k)),
    sigmoid(beta_logits) [B,H,T] or None); beta_logits [B,1,T] (shared by all
    heads) or [B,H,T].  out = (q_out, k_out) may be given (they may be q, k)."""
    B, H, T, dk = q.shape
    dev, dtype = _inputs("deltanet_prologue", dict(q=q, k=k), dict(q=(B, H, T, dk), k=(B, H, T, dk)))
    bh = 1
    if beta_logits is not None:
        if beta_logits.dim() != 3 or beta_logits.shape[0] != B or beta_logits.shape[2] != T:
            raise ValueError("deltanet_prologue: beta_logits must be [B,1,T] or [B,H,T]")
        bh = beta_logits.shape[1]
        _inputs("deltanet_prologue", dict(q=q, beta_logits=beta_logits),
                dict(q=(B, H, T, dk), beta_logits=(B, bh, T)))
    qo, ko = out if out is not None else (torch.empty_like(q), torch.empty_like(k))
    _out("deltanet_prologue", qo, (B, H, T, dk), dev, dtype)
    _out("deltanet_prologue", ko, (B, H, T, dk), dev, dtype)
    bo = torch.empty(B, H, T, device=dev, dtype=dtype) if beta_logits is not None else None
    rc = library().deltanet_prologue(_ptr(q), _ptr(k), _ptr(beta_logits), _ptr(qo), _ptr(ko),
                                     _ptr(bo), B, H, T, dk, bh, int(bool(apply_silu)),
                                     float(q_scale), _DTYPES[dtype], _stream(dev, stream))
    _check("deltanet_prologue", rc)
    return qo, ko, bo
