"""The sequence-parallel chunk-state scan prototype
(delta_rule_recurrent_chunkwise_amd/segmented.py): the sequence cut into P
segments, each run from zero and from the identity through the library's
prefill, the incoming states scanned and the outputs corrected.  The result
must equal the oracle's per-token recurrence over the whole sequence, for the
delta rule without a gate, with a per-key-channel gate and with one decay per
token, with and without an initial state, for segment lengths that are and
are not whole chunks."""
import pytest
import torch

import oracle
import workloads
from delta_rule_recurrent_chunkwise_amd.segmented import segmented_delta_prefill
from gpu_common import TOL, assert_close, require_gpu

pytestmark = pytest.mark.gpu

GATES = [False, True, "token"]
GATE_IDS = ["no-gate", "per-channel", "per-token"]


@pytest.mark.parametrize("init", [False, True], ids=["zero", "init"])
@pytest.mark.parametrize("gated", GATES, ids=GATE_IDS)
@pytest.mark.parametrize("T,P", [(1024, 2), (1024, 4), (1024, 8), (960, 3)],
                         ids=["T1024-P2", "T1024-P4", "T1024-P8", "T960-P3"])
def test_segmented_equals_the_recurrence(T, P, gated, init):
    dev = require_gpu()
    B, H, d = 1, 3, 128
    print(f"segmented prefill T={T} P={P} gate={gated} init={init}", flush=True)
    inp = workloads.make_delta(B, H, T, d, d, torch.bfloat16, seed=800 + T + P, gated=gated,
                               init_state=init, state_std=0.5)
    x = {k: v.to(dev) for k, v in inp.items()}
    o, S = segmented_delta_prefill(x["q"], x["k"], x["v"], x["beta"], P, g=x.get("g"),
                                   token_gate=(gated == "token"),
                                   S0=x["S0"] if init else None)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.delta_recurrent(inp["q"], inp["k"], inp["v"], inp["beta"],
                                          inp.get("g"), S0=inp["S0"] if init else None)
    assert_close(o, o_ref, TOL[torch.bfloat16], "o")
    assert_close(S, S_ref, TOL[torch.bfloat16], "S")


def test_segmented_rejects_a_ragged_split():
    dev = require_gpu()
    inp = workloads.make_delta(1, 1, 100, 128, 128, torch.bfloat16, seed=7)
    x = {k: v.to(dev) for k, v in inp.items()}
    with pytest.raises(ValueError):
        segmented_delta_prefill(x["q"], x["k"], x["v"], x["beta"], 3)
