"""la_prefill_noalloc, the entry point for callers that cannot allocate,
against la_prefill (the same kernels with a caller workspace): two calls in a
row through the C ABI, the second smaller, on the library's fixed scratch."""
import pytest
import torch

import delta_rule_recurrent_chunkwise_amd as la
import workloads
from gpu_common import TOL, assert_close, require_gpu

pytestmark = pytest.mark.gpu


def _pair(B, H, T, dk, dv, dtype, seed, init):
    dev = require_gpu()
    inp = workloads.make_la(B, H, T, dk, dv, dtype, seed=seed, init_state=init)
    d = {n: t.to(dev) for n, t in inp.items()}
    S_ref = d["S0"].clone() if init else None
    z_ref = d["z0"].clone() if init else None
    o_ref, S_ref, z_ref = la.la_prefill(d["q"], d["k"], d["v"], S=S_ref, z=z_ref,
                                        use_initial_state=init)
    o = torch.empty(B, H, T, dv, device=dev, dtype=dtype)
    S = d["S0"].clone() if init else torch.empty(B, H, dk, dv, device=dev)
    z = d["z0"].clone() if init else torch.empty(B, H, dk, device=dev)
    torch.cuda.synchronize()
    # torch's count of allocation requests so far (frees, e.g. by garbage
    # collection of earlier tests' tensors, do not change it)
    before = torch.cuda.memory_stats(dev)["allocation.all.allocated"]
    la.la_prefill_noalloc(d["q"], d["k"], d["v"], o, S, z, use_initial_state=init)
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats(dev)["allocation.all.allocated"] == before, \
        "the call allocated through torch"
    return (o, S, z), (o_ref, S_ref, z_ref)


def test_noalloc_matches_la_prefill_twice_second_smaller():
    print("la_prefill_noalloc: B=8 H=12 T=1024 d=64 bf16, then B=2 H=3 T=200 dk=32 dv=64",
          flush=True)
    need = la.la_prefill_workspace_bytes(8, 12, 1024, 64, 64, torch.bfloat16)
    assert 0 < need <= la.NOALLOC_SCRATCH_BYTES
    for (B, H, T, dk, dv, seed, init) in ((8, 12, 1024, 64, 64, 71, False),
                                          (2, 3, 200, 32, 64, 72, True)):
        got, ref = _pair(B, H, T, dk, dv, torch.bfloat16, seed, init)
        for name, g, r in zip(("o", "S", "z"), got, ref):
            assert_close(g, r, TOL[torch.bfloat16], f"{name} B={B} H={H} T={T}")
            # the same kernels on the same inputs: the same bits
            assert torch.equal(g, r), name


def test_noalloc_float32_needs_no_scratch():
    print("la_prefill_noalloc: float32 B=1 H=2 T=100 d=16", flush=True)
    assert la.la_prefill_workspace_bytes(1, 2, 100, 16, 16, torch.float32) == 0
    got, ref = _pair(1, 2, 100, 16, 16, torch.float32, 73, False)
    for name, g, r in zip(("o", "S", "z"), got, ref):
        assert_close(g, r, TOL[torch.float32], name)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    dev = require_gpu()
    B, H, T, d = 8, 12, 4096, 64     # 152 MB of per-chunk states
    assert la.la_prefill_workspace_bytes(B, H, T, d, d, torch.bfloat16) > la.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, H, T, d, device=dev, dtype=torch.bfloat16)
    o = torch.empty_like(q)
    S = torch.empty(B, H, d, d, device=dev)
    z = torch.empty(B, H, d, device=dev)
    with pytest.raises(la.LinAttnError) as e:
        la.la_prefill_noalloc(q, q, q, o, S, z)
    assert e.value.code == -8
