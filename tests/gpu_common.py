"""Shared helpers for the GPU parity tests: tolerances and the comparison
metric max|gpu - ref| / max|ref| (over the whole compared tensor)."""
import json
import os

import numpy as np
import pytest
import torch

# float32 inputs: 1e-4; bf16 inputs (fp32 state, bf16 MFMA operands): 2e-2
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    return torch.device("cuda:0")


def to64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, np.float64)


def rel_err(gpu, ref) -> float:
    g, r = to64(gpu), to64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    scale = float(np.max(np.abs(r)))
    if scale == 0.0:
        scale = 1.0
    diff = np.abs(g - r)
    if not np.all(np.isfinite(g)):
        return float("inf")
    return float(np.max(diff)) / scale


def _log_margin(what, err, tol):
    """Append the achieved error to the JSON-lines file named by the
    environment variable LINATTN_PARITY_LOG (if set), so a run records its
    margins under the tolerance, not just pass/fail."""
    path = os.environ.get("LINATTN_PARITY_LOG")
    if not path:
        return
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    with open(path, "a") as f:
        f.write(json.dumps({"test": test, "what": what, "rel_err": err, "tol": tol}) + "\n")


def assert_close(gpu, ref, tol, what):
    err = rel_err(gpu, ref)
    print(f"  {what}: rel err {err:.3e} (tol {tol:.0e})", flush=True)
    _log_margin(what, err, tol)
    assert err <= tol, f"{what}: max|gpu-ref|/max|ref| = {err:.3e} > {tol:.1e}"
