"""The C ABI of liblinattn.so without a GPU: the library loads, exports every
function include/linattn.h declares, and rejects bad arguments with the
documented codes before making any HIP call (the pointers passed here are
never dereferenced)."""
import ctypes
import os
import re

import pytest

import delta_rule_recurrent_chunkwise_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linattn.h")

OK, NULL, SHAPE, DTYPE, DIM, LAUNCH, ALIGN, WORKSPACE = 0, -1, -2, -3, -4, -5, -6, -7
P = ctypes.c_void_p
FAKE = P(0x1000)          # 256-byte aligned, never dereferenced
MISALIGNED = P(0x1002)
BIG = 1 << 40             # a workspace size no call here needs more than


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def _codes():
    text = open(HEADER).read()
    return {m[0]: int(m[1]) for m in re.findall(r"#define\s+(LA_\w+)\s+\(?(-?\d+)\)?", text)}


def test_library_loads_and_exports_every_declared_symbol():
    lib = la.library()
    declared = _declared_functions()
    assert set(declared) == set(la.EXPORTED_SYMBOLS), declared
    for name in declared:
        assert hasattr(lib, name), f"{name} not exported"


def test_error_codes_match_header():
    codes = _codes()
    assert codes["LA_OK"] == OK and codes["LA_ERR_NULL"] == NULL
    assert codes["LA_ERR_SHAPE"] == SHAPE and codes["LA_ERR_DTYPE"] == DTYPE
    assert codes["LA_ERR_UNSUPPORTED_DIM"] == DIM and codes["LA_ERR_LAUNCH"] == LAUNCH
    assert codes["LA_ERR_ALIGN"] == ALIGN and codes["LA_ERR_WORKSPACE"] == WORKSPACE
    assert codes["LA_DTYPE_F32"] == 0 and codes["LA_DTYPE_BF16"] == 1


def test_strerror_is_static_text_for_every_code():
    for code in (OK, NULL, SHAPE, DTYPE, DIM, LAUNCH, ALIGN, WORKSPACE, -99, 7):
        msg = la.la_strerror(code)
        assert isinstance(msg, str) and msg
    assert la.la_strerror(-99) == "unknown error code"


def _la_prefill(q=FAKE, k=FAKE, v=FAKE, o=FAKE, S=FAKE, z=FAKE, init=0, B=1, H=1, T=64,
                dk=64, dv=64, dt=1, ws=FAKE, wsn=BIG):
    return la.library().la_prefill(q, k, v, o, S, z, init, B, H, T, dk, dv, dt, ws, wsn, None)


def _la_decode(q=FAKE, k=FAKE, v=FAKE, o=FAKE, S=FAKE, z=FAKE, N=1, H=1, dk=64, dv=64, dt=1):
    return la.library().la_decode_step(q, k, v, o, S, z, N, H, dk, dv, dt, None)


def _dn_prefill(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=None, o=FAKE, S=FAKE, init=0, B=1, H=1,
                T=64, dk=64, dv=64, dt=1, ws=FAKE, wsn=BIG):
    return la.library().deltanet_prefill(q, k, v, beta, g, o, S, init, B, H, T, dk, dv, dt,
                                         ws, wsn, None)


def _dn_decode(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=None, o=FAKE, S=FAKE, N=1, H=1, dk=64,
               dv=64, dt=1):
    return la.library().deltanet_decode_step(q, k, v, beta, g, o, S, N, H, dk, dv, dt, None)


def _gdn_prefill(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=FAKE, o=FAKE, S=FAKE, init=0, B=1, H=1,
                 T=64, dk=64, dv=64, dt=1):
    return la.library().gated_deltanet_prefill(q, k, v, beta, g, o, S, init, B, H, T, dk, dv,
                                               dt, None)


def _gdn_decode(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=FAKE, o=FAKE, S=FAKE, N=1, H=1, dk=64,
                dv=64, dt=1):
    return la.library().gated_deltanet_decode_step(q, k, v, beta, g, o, S, N, H, dk, dv, dt,
                                                   None)


def _gla_prefill(q=FAKE, k=FAKE, v=FAKE, g=FAKE, o=FAKE, S=FAKE, init=0, B=1, H=1, T=64,
                 dk=64, dv=64, dt=1, ws=FAKE, wsn=BIG):
    return la.library().gla_prefill(q, k, v, g, o, S, init, B, H, T, dk, dv, dt, ws, wsn, None)


def _gla_decode(q=FAKE, k=FAKE, v=FAKE, g=FAKE, o=FAKE, S=FAKE, N=1, H=1, dk=64, dv=64, dt=1):
    return la.library().gla_decode_step(q, k, v, g, o, S, N, H, dk, dv, dt, None)


@pytest.mark.parametrize("missing", ["q", "k", "v", "beta", "g", "o", "S"])
def test_gated_deltanet_null_pointers(missing):
    assert _gdn_prefill(**{missing: None}) == NULL
    assert _gdn_decode(**{missing: None}) == NULL


@pytest.mark.parametrize("missing", ["q", "k", "v", "o", "S"])
def test_gla_null_pointers(missing):
    """g may be NULL (no decay); everything else is required."""
    assert _gla_prefill(**{missing: None}) == NULL
    assert _gla_decode(**{missing: None}) == NULL


def test_scalar_gated_entry_points_validate_like_the_others():
    for fn in (_gdn_prefill, _gla_prefill):
        assert fn(dt=5) == DTYPE
        assert fn(T=-1) == SHAPE
        assert fn(B=0) == SHAPE
        assert fn(dk=96) == DIM
        assert fn(q=MISALIGNED) == ALIGN
        assert fn(o=MISALIGNED) == ALIGN
    for fn in (_gdn_decode, _gla_decode):
        assert fn(dt=5) == DTYPE
        assert fn(N=0) == SHAPE
        assert fn(dv=8) == DIM
        assert fn(S=MISALIGNED) == ALIGN
    none = dict(q=None, k=None, v=None, o=None)
    assert _gdn_prefill(T=0, init=1, beta=None, g=None, **none) == OK
    assert _gla_prefill(T=0, init=1, g=None, **none) == OK


def _bwd(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, S0=None, dO=FAKE, dST=None, dq=FAKE, dk_=FAKE,
         dv_=FAKE, db=FAKE, dS0=None, B=1, H=1, T=64, dk=64, dv=64, dt=1, ws=FAKE, wsn=BIG):
    return la.library().deltanet_prefill_backward(q, k, v, beta, S0, dO, dST, dq, dk_, dv_, db,
                                                  dS0, B, H, T, dk, dv, dt, ws, wsn, None)


def _pro(qi=FAKE, ki=FAKE, bl=None, qo=FAKE, ko=FAKE, bo=None, B=1, H=2, T=64, dk=64, bh=1,
         silu=1, scale=1.0, dt=1):
    return la.library().deltanet_prologue(qi, ki, bl, qo, ko, bo, B, H, T, dk, bh, silu,
                                          ctypes.c_float(scale), dt, None)


@pytest.mark.parametrize("missing", ["q", "k", "v", "beta", "dO", "dq", "dk_", "dv_", "db"])
def test_backward_null_pointers(missing):
    assert _bwd(**{missing: None}) == NULL


def test_backward_validation():
    assert _bwd(dt=3) == DTYPE
    assert _bwd(T=-1) == SHAPE
    assert _bwd(dk=96) == DIM
    assert _bwd(dt=0, dk=128) == DIM    # float32 backward: dk, dv <= 64
    assert _bwd(dt=0, dv=128) == DIM
    assert _bwd(dO=MISALIGNED) == ALIGN
    assert _bwd(q=MISALIGNED) == ALIGN
    for out in ("dq", "dk_", "dv_"):  # written in 8- and 16-byte vectors
        assert _bwd(**{out: MISALIGNED}) == ALIGN
    assert _bwd(db=MISALIGNED) != ALIGN  # dbeta is written element by element


def _gbwd(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=FAKE, S0=None, dO=FAKE, dST=None, dq=FAKE,
          dk_=FAKE, dv_=FAKE, db=FAKE, dg=FAKE, dS0=None, B=1, H=1, T=64, dk=64, dv=64, dt=1,
          ws=FAKE, wsn=BIG):
    return la.library().gated_deltanet_prefill_backward(q, k, v, beta, g, S0, dO, dST, dq, dk_,
                                                        dv_, db, dg, dS0, B, H, T, dk, dv, dt,
                                                        ws, wsn, None)


@pytest.mark.parametrize("missing", ["q", "k", "v", "beta", "g", "dO", "dq", "dk_", "dv_", "db",
                                     "dg"])
def test_gated_backward_null_pointers(missing):
    assert _gbwd(**{missing: None}) == NULL


def test_gated_backward_validation():
    assert _gbwd(dt=3) == DTYPE
    assert _gbwd(T=-1) == SHAPE
    assert _gbwd(dv=96) == DIM
    assert _gbwd(dt=0, dk=128) == DIM   # float32: dk, dv <= 64, as without a gate
    assert _gbwd(dO=MISALIGNED) == ALIGN
    for out in ("dq", "dk_", "dv_"):
        assert _gbwd(**{out: MISALIGNED}) == ALIGN
    assert _gbwd(dg=MISALIGNED) != ALIGN  # dg is written element by element


def _kbwd(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=FAKE, S0=None, dO=FAKE, dST=None, dq=FAKE,
          dk_=FAKE, dv_=FAKE, db=FAKE, dg=FAKE, dS0=None, B=1, H=1, T=64, dk=64, dv=64, dt=1,
          ws=FAKE, wsn=BIG):
    return la.library().kda_prefill_backward(q, k, v, beta, g, S0, dO, dST, dq, dk_, dv_, db, dg,
                                             dS0, B, H, T, dk, dv, dt, ws, wsn, None)


@pytest.mark.parametrize("missing", ["q", "k", "v", "beta", "g", "dO", "dq", "dk_", "dv_", "db",
                                     "dg"])
def test_kda_backward_null_pointers(missing):
    assert _kbwd(**{missing: None}) == NULL


def test_kda_backward_validation():
    assert _kbwd(dt=3) == DTYPE
    assert _kbwd(T=-1) == SHAPE
    assert _kbwd(dk=96) == DIM
    assert _kbwd(dt=0) == DIM           # bf16 only
    assert _kbwd(dt=0, dk=16, dv=16) == DIM
    assert _kbwd(dO=MISALIGNED) == ALIGN
    for out in ("dq", "dk_", "dv_"):
        assert _kbwd(**{out: MISALIGNED}) == ALIGN
    assert _kbwd(ws=None, wsn=0) == WORKSPACE
    assert _kbwd(wsn=la.kda_prefill_backward_workspace_bytes(1, 1, 64, 64, 64, 1) - 1) == WORKSPACE


@pytest.mark.parametrize("missing", ["qi", "ki", "qo", "ko"])
def test_prologue_null_pointers(missing):
    assert _pro(**{missing: None}) == NULL


def test_prologue_validation():
    assert _pro(bl=FAKE) == NULL             # beta logits without an output
    assert _pro(bo=FAKE) == NULL
    assert _pro(bl=FAKE, bo=FAKE, bh=3) == SHAPE   # beta heads must be 1 or H
    assert _pro(dt=2) == DTYPE
    assert _pro(B=0) == SHAPE
    assert _pro(dk=48) == DIM
    assert _pro(qo=MISALIGNED) == ALIGN
    assert _pro(T=0, qi=None, ki=None, qo=None, ko=None) == OK   # nothing to do, no HIP call


@pytest.mark.parametrize("missing", ["q", "k", "v", "o", "S", "z"])
def test_la_null_pointers(missing):
    assert _la_prefill(**{missing: None}) == NULL
    assert _la_decode(**{missing: None}) == NULL


@pytest.mark.parametrize("missing", ["q", "k", "v", "beta", "o", "S"])
def test_deltanet_null_pointers(missing):
    assert _dn_prefill(**{missing: None}) == NULL
    assert _dn_decode(**{missing: None}) == NULL


@pytest.mark.parametrize("dt", [-1, 2, 7])
def test_bad_dtype(dt):
    assert _la_prefill(dt=dt) == DTYPE
    assert _la_decode(dt=dt) == DTYPE
    assert _dn_prefill(dt=dt) == DTYPE
    assert _dn_decode(dt=dt) == DTYPE


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(B=-3), dict(T=-1), dict(T=-64),
                                dict(T=2**31 - 1), dict(B=1 << 16, H=1 << 10, T=1 << 14)])
def test_bad_prefill_shape(kw):
    assert _la_prefill(**kw) == SHAPE
    assert _dn_prefill(**kw) == SHAPE


def test_empty_prefill_with_initial_state_is_a_no_op():
    """T = 0 with the initial state kept enqueues nothing (no HIP call, so it
    runs here) and accepts NULL token arrays; S and z are required."""
    none = dict(q=None, k=None, v=None, o=None)
    assert _la_prefill(T=0, init=1, **none) == OK
    assert _dn_prefill(T=0, init=1, beta=None, **none) == OK
    assert _la_prefill(T=0, init=1, S=None) == NULL
    assert _la_prefill(T=0, init=1, z=None) == NULL
    assert _dn_prefill(T=0, init=1, S=None) == NULL


@pytest.mark.parametrize("kw", [dict(N=0), dict(H=0), dict(N=-1), dict(N=1 << 20, H=1 << 12)])
def test_bad_decode_shape(kw):
    assert _la_decode(**kw) == SHAPE
    assert _dn_decode(**kw) == SHAPE


@pytest.mark.parametrize("kw", [dict(dk=8), dict(dv=8), dict(dk=96), dict(dv=256),
                                dict(dk=0), dict(dv=-16)])
def test_unsupported_dims(kw):
    expected = SHAPE if min(kw.values()) <= 0 else DIM
    got = {_la_prefill(**kw), _la_decode(**kw), _dn_prefill(**kw), _dn_decode(**kw)}
    assert got <= {DIM, SHAPE} and (DIM in got if expected == DIM else True)


def test_float32_gated_prefill_limited_to_dk_64():
    assert _dn_prefill(g=FAKE, dt=0, dk=128, dv=64) == DIM


def test_misaligned_vector_pointers():
    assert _la_prefill(q=MISALIGNED) == ALIGN
    assert _dn_prefill(v=MISALIGNED) == ALIGN
    assert _la_prefill(o=MISALIGNED) == ALIGN  # outputs are written in vectors too
    assert _dn_prefill(o=MISALIGNED) == ALIGN
    assert _la_decode(S=MISALIGNED) == ALIGN
    assert _dn_decode(S=MISALIGNED) == ALIGN


def test_python_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 64, 16)
    with pytest.raises(ValueError):
        la.deltanet_prefill(q, q, q, torch.zeros(1, 1, 64))
    with pytest.raises(ValueError):
        la.la_prefill(q, q, q)


def test_peak_probe_library_loads_and_rejects_bad_arguments():
    """The measurement harness's peak probes (libpeak_probe.so, not part of the
    linattn ABI) check their arguments before any launch."""
    path = os.path.join(ROOT, "delta_rule_recurrent_chunkwise_amd", "libpeak_probe.so")
    if not os.path.exists(path):
        pytest.skip("libpeak_probe.so not built")
    lib = ctypes.CDLL(path)
    lib.peak_probe_mfma_bf16.argtypes = [P, P, ctypes.c_int, ctypes.c_int, P]
    lib.peak_probe_stream.argtypes = [P, P, ctypes.c_size_t, ctypes.c_int, P]
    assert lib.peak_probe_mfma_bf16(None, FAKE, 1, 1, None) == -1
    assert lib.peak_probe_mfma_bf16(FAKE, FAKE, 0, 1, None) == -1
    assert lib.peak_probe_mfma_bf16(FAKE, FAKE, 1, 0, None) == -1
    assert lib.peak_probe_stream(None, FAKE, 1 << 15, 0, None) == -1
    assert lib.peak_probe_stream(FAKE, None, 1 << 15, 0, None) == -1      # copy needs dst
    assert lib.peak_probe_stream(FAKE, FAKE, (1 << 15) + 16, 0, None) == -1  # not whole tiles
    assert lib.peak_probe_stream(MISALIGNED, FAKE, 1 << 15, 1, None) == -1


# ---------------------------------------------------------------------------
# Workspaces: the library allocates nothing; the entry points that need scratch
# memory take it from the caller and check it before any HIP call.
# ---------------------------------------------------------------------------
def _nch(T):
    return (T + 63) // 64


def test_workspace_queries_match_the_documented_sizes():
    B, H, T = 2, 3, 130
    C = _nch(T)
    for dk, dv in ((16, 32), (64, 64), (128, 128)):
        la_ws = 6 * B * H * C * dk * dv + 4 * B * H * C * dk
        assert la.la_prefill_workspace_bytes(B, H, T, dk, dv, 1) == la_ws
        assert la.gla_prefill_workspace_bytes(B, H, T, dk, dv, 1) == la_ws
        assert la.la_prefill_workspace_bytes(B, H, T, dk, dv, 0) == 0    # float32: one kernel
        assert la.deltanet_prefill_workspace_bytes(0, B, H, T, dk, dv, 1) == 0
        assert la.deltanet_prefill_workspace_bytes(1, B, H, T, dk, dv, 0) == 0
        gated = 384 * B * H * C * dk + 4 * B * H * C * dk if dk == 128 and dv % 32 == 0 else 0
        assert la.deltanet_prefill_workspace_bytes(1, B, H, T, dk, dv, 1) == gated

        def r(n):
            return (n + 255) // 256 * 256
        nst = B * H * C * dk * dv
        bwd = 2 * r(4 * nst) + r(2 * B * H * C * dk * (dk + 64))
        assert la.deltanet_prefill_backward_workspace_bytes(B, H, T, dk, dv, 1) == bwd
        assert la.gated_deltanet_prefill_backward_workspace_bytes(B, H, T, dk, dv, 1) == \
            bwd + r(4 * B * H * C)
        kda = r(388 * B * H * C * dk) + 2 * r(2 * nst) + r(2 * B * H * C * dk * (dk + 64))
        assert la.kda_prefill_backward_workspace_bytes(B, H, T, dk, dv, 1) == kda
        assert la.kda_prefill_backward_workspace_bytes(B, H, T, dk, dv, 0) == 0  # bf16 only
    assert la.deltanet_prefill_backward_workspace_bytes(B, H, T, 64, 64, 0) == 2 * 4 * B * H * C * 64 * 64


def test_workspace_queries_are_zero_when_nothing_runs_or_the_call_is_invalid():
    for q in (la.la_prefill_workspace_bytes, la.gla_prefill_workspace_bytes,
              la.deltanet_prefill_backward_workspace_bytes,
              la.gated_deltanet_prefill_backward_workspace_bytes,
              la.kda_prefill_backward_workspace_bytes):
        assert q(1, 1, 0, 64, 64, 1) == 0          # T = 0
        assert q(0, 1, 64, 64, 64, 1) == 0         # bad shape
        assert q(1, 1, 64, 96, 64, 1) == 0         # bad dim
        assert q(1, 1, 64, 64, 64, 5) == 0         # bad dtype
    assert la.deltanet_prefill_backward_workspace_bytes(1, 1, 64, 128, 64, 0) == 0  # fp32 dk 128


def test_missing_or_small_workspace_is_rejected_before_any_hip_call():
    need = la.la_prefill_workspace_bytes(1, 1, 64, 64, 64, 1)
    assert need > 0
    assert _la_prefill(ws=None, wsn=0) == WORKSPACE
    assert _la_prefill(ws=None, wsn=BIG) == WORKSPACE
    assert _la_prefill(wsn=need - 1) == WORKSPACE
    assert _la_prefill(ws=P(0x1010), wsn=BIG) == ALIGN          # 16- but not 256-byte aligned
    assert _gla_prefill(ws=None, wsn=0) == WORKSPACE
    assert _gla_prefill(wsn=la.gla_prefill_workspace_bytes(1, 1, 64, 64, 64, 1) - 1) == WORKSPACE
    assert _dn_prefill(g=FAKE, dk=128, dv=128, ws=None, wsn=0) == WORKSPACE
    assert _dn_prefill(g=FAKE, dk=128, dv=128,
                       wsn=la.deltanet_prefill_workspace_bytes(1, 1, 1, 64, 128, 128, 1) - 1) == WORKSPACE
    assert _bwd(ws=None, wsn=0) == WORKSPACE
    assert _bwd(wsn=la.deltanet_prefill_backward_workspace_bytes(1, 1, 64, 64, 64, 1) - 1) == WORKSPACE
    assert _gbwd(ws=None, wsn=0) == WORKSPACE
    assert _gbwd(wsn=la.gated_deltanet_prefill_backward_workspace_bytes(1, 1, 64, 64, 64, 1) - 1) \
        == WORKSPACE
    # earlier checks win: a bad call is reported as such even without a workspace
    assert _la_prefill(dt=7, ws=None, wsn=0) == DTYPE
    assert _la_prefill(q=None, ws=None, wsn=0) == NULL
    assert _la_prefill(q=MISALIGNED, ws=None, wsn=0) == ALIGN


def test_paths_without_a_workspace_accept_none():
    """No workspace is needed (or read) where the query returns 0: the
    ungated delta rule and float32 linear attention reach their launch, which
    cannot happen here, so only T = 0 (no HIP call) is run through."""
    none = dict(q=None, k=None, v=None, o=None)
    assert _la_prefill(T=0, init=1, ws=None, wsn=0, **none) == OK
    assert _dn_prefill(T=0, init=1, beta=None, ws=None, wsn=0, **none) == OK
    assert _gla_prefill(T=0, init=1, g=None, ws=None, wsn=0, **none) == OK


def test_no_allocation_calls_in_the_library_sources():
    """The library allocates no device memory: no hipMalloc / hipFree of any
    kind appears in its sources."""
    csrc = os.path.join(ROOT, "delta_rule_recurrent_chunkwise_amd", "csrc")
    for name in os.listdir(csrc):
        if name.endswith((".hip", ".hpp")) and name != "peak_probe.hip":
            text = open(os.path.join(csrc, name)).read()
            assert not re.search(r"hip(Malloc|Free|ExtMalloc|HostMalloc)", text), name


def test_noalloc_checks_its_limit_before_any_hip_call():
    """la_prefill_noalloc validates like la_prefill and rejects sizes beyond
    its fixed scratch with LA_ERR_SCRATCH_LIMIT, all before any HIP call."""
    lib = la.library()

    def call(q=FAKE, o=FAKE, S=FAKE, z=FAKE, B=1, H=1, T=64, dk=64, dv=64, dt=1):
        return lib.la_prefill_noalloc(q, FAKE, FAKE, o, S, z, 0, B, H, T, dk, dv, dt, None)
    assert _codes()["LA_ERR_SCRATCH_LIMIT"] == -8
    assert call(B=8, H=12, T=4096) == -8          # 152 MB > 64 MiB
    assert call(B=64, H=64, T=1 << 14, dk=128, dv=128) == -8
    assert call(q=None) == NULL and call(S=None) == NULL and call(z=None) == NULL
    assert call(dt=4) == DTYPE and call(B=0) == SHAPE and call(T=-1) == SHAPE
    assert call(dk=96) == DIM and call(q=MISALIGNED) == ALIGN


def _seg(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=None, gate=0, o=FAKE, S=FAKE, init=0, B=1, H=1,
         T=1024, dk=64, dv=64, dt=1, segs=4, ws=FAKE, wsn=BIG):
    return la.library().deltanet_prefill_segmented(q, k, v, beta, g, gate, o, S, init, B, H, T, dk,
                                                   dv, dt, segs, ws, wsn, None)


@pytest.mark.parametrize("missing", ["q", "k", "v", "beta", "o", "S"])
def test_segmented_null_pointers(missing):
    assert _seg(**{missing: None}) == NULL
    assert _seg(g=FAKE, gate=1, **{missing: None}) == NULL


def test_segmented_validation():
    assert _seg(gate=1) == NULL                   # a gate without g
    assert _seg(gate=2) == NULL
    assert _seg(g=FAKE) == SHAPE                  # g without a gate
    assert _seg(g=FAKE, gate=3) == SHAPE
    assert _seg(g=FAKE, gate=-1) == SHAPE
    assert _seg(dt=3) == DTYPE
    assert _seg(B=0) == SHAPE
    assert _seg(segs=-1) == SHAPE
    assert _seg(segs=3) == SHAPE                  # 1024 % 3 != 0
    assert _seg(segs=2048) == SHAPE               # more segments than tokens
    assert _seg(dk=96) == DIM
    assert _seg(dt=0) == DIM                      # bf16 only
    assert _seg(dt=0, segs=1) == DIM
    for p in ("q", "k", "v", "o"):
        assert _seg(**{p: MISALIGNED}) == ALIGN
    need = la.deltanet_prefill_segmented_workspace_bytes(None, 1, 1, 1024, 64, 64, 1, 4)
    assert need > 0
    assert _seg(ws=None, wsn=0) == WORKSPACE
    assert _seg(wsn=need - 1) == WORKSPACE
    assert _seg(ws=P(0x1010)) == ALIGN


def test_segmented_workspace_formula():
    def r(n):
        return (n + 255) // 256 * 256

    for B, H, T, dk, dv, P in ((1, 4, 32768, 128, 128, 16), (2, 3, 1000, 64, 32, 8),
                               (1, 1, 96, 16, 128, 3), (3, 2, 640, 128, 64, 5)):
        n, Tp, k32 = B * H * P, T // P, (dk + 31) // 32
        base = (r(4 * n * dk * dv) + r(4 * n * dk * dk) + 2 * r(2 * n * Tp * dk)
                + r(128 * B * H * (P - 1) * k32 * dv) + r(128 * n * dk * k32))
        for gate in (None, "token"):
            assert la.deltanet_prefill_segmented_workspace_bytes(gate, B, H, T, dk, dv, 1, P) == base
        prep = max(la.deltanet_prefill_workspace_bytes(True, B, H * P, Tp, dk, dv, 1),
                   la.deltanet_prefill_workspace_bytes(True, B, H * P, Tp, dk, dk, 1))
        assert la.deltanet_prefill_segmented_workspace_bytes("channel", B, H, T, dk, dv, 1, P) == \
            base + r(prep)
        assert la.deltanet_prefill_segmented_workspace_bytes(None, B, H, T, dk, dv, 0, P) == 0
    # one segment: the one-pass entry points' workspace
    assert la.deltanet_prefill_segmented_workspace_bytes(None, 1, 32, 4096, 128, 128, 1, 1) == 0
    assert la.deltanet_prefill_segmented_workspace_bytes("channel", 1, 32, 4096, 128, 128, 1, 1) == \
        la.deltanet_prefill_workspace_bytes(True, 1, 32, 4096, 128, 128, 1)
    assert la.deltanet_prefill_segmented_workspace_bytes(None, 1, 1, 0, 64, 64, 1, 4) == 0  # T = 0
    assert la.deltanet_prefill_segmented_workspace_bytes(None, 1, 1, 100, 64, 64, 1, 3) == 0  # 100 % 3


def test_segment_count_rule():
    """The automatic segment count: the largest power of two P <= 64 with
    B*H*P*ceil(dv/32) <= 256, T % P == 0 and T/P >= 512, else 1 when below 4."""
    seg = la.deltanet_prefill_segments
    assert seg(1, 4, 32768, 128, 128) == 16
    assert seg(1, 8, 32768, 128, 128) == 8
    assert seg(1, 16, 32768, 128, 128) == 4
    assert seg(1, 32, 32768, 128, 128) == 1      # two segments would not pay
    assert seg(4, 16, 4096, 128, 128) == 1
    assert seg(1, 4, 4096, 128, 128) == 8        # T / 16 = 256 tokens is too short
    assert seg(1, 1, 65536, 64, 16) == 64
    assert seg(2, 3, 3000, 128, 128) == 4        # T / 8 = 375 is too short
    assert seg(1, 1, 100, 64, 64) == 1
    assert seg(0, 1, 100, 64, 64) == 0           # invalid
    assert seg(1, 1, 100, 96, 64) == 0
