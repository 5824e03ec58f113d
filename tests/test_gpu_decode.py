"""GPU parity of kda_recurrent_step against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_12_amd as kda
import oracle
import synth
from tests.helpers import check_close, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
ODT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _cuda(d):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("act,out", [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16")])
def test_decode_steps_small(Dk, Dv, act, out):
    print(f"[decode small Dk={Dk} Dv={Dv} act={act} out={out}]", flush=True)
    steps = 6
    inp = _cuda(synth.decode_inputs(5, 3, Dk, Dv, steps, act, mu=-2.0, s0_std=0.02, seed=11))
    state = inp["state"].clone()
    st_ref = to_np(inp["state"])
    for s in range(steps):
        o = kda.kda_recurrent_step(inp["q"][s], inp["k"][s], inp["v"][s], inp["alpha"][s],
                                   inp["beta"][s], state, out_dtype=ODT[out])
        torch.cuda.synchronize()
        o_ref, st_ref = oracle.kda_step(to_np(inp["q"][s]), to_np(inp["k"][s]), to_np(inp["v"][s]),
                                        to_np(inp["alpha"][s]), to_np(inp["beta"][s]), st_ref)
        if out == "f32":
            check_close(o, o_ref, "f32", what=f"o step {s}")
        else:
            check_close(o, o_ref, "bf16", stored_bf16=True, what=f"o step {s}")
    check_close(state, st_ref, "f32", what="state")


def test_decode_readback_overwrite():
    # beta = 1, unit keys, q = k: the decayed-then-overwritten memory returns v
    # exactly (up to fp32 rounding) -- the delta rule's erase-then-write.
    print("[decode readback]", flush=True)
    inp = _cuda(synth.decode_inputs(8, 4, 128, 128, 1, "f32", mu=-1.0, s0_std=0.5, seed=3))
    state = inp["state"].clone()
    o = kda.kda_recurrent_step(inp["k"][0], inp["k"][0], inp["v"][0], inp["alpha"][0],
                               torch.ones_like(inp["beta"][0]), state)
    torch.cuda.synchronize()
    assert torch.allclose(o, inp["v"][0], atol=2e-5, rtol=0)


def test_decode_full_workload():
    """256 sequences x 32 heads, d=128, 100 in-place steps (the decode benchmark
    launch): every step's whole output and the whole final state are compared
    with the oracle run step by step on all 8192 (sequence, head) pairs."""
    w = synth.WORKLOADS[3]
    print(f"[decode full {w.name}]", flush=True)
    inp = synth.workload_inputs(3, device=DEV)
    state = inp["state"].clone()
    st = to_np(inp["state"])
    worst = 0.0
    for s in range(w.steps):
        o = kda.kda_recurrent_step(inp["q"][s], inp["k"][s], inp["v"][s], inp["alpha"][s],
                                   inp["beta"][s], state, out_dtype=torch.bfloat16)
        o_ref, st = oracle.kda_step(to_np(inp["q"][s]), to_np(inp["k"][s]), to_np(inp["v"][s]),
                                    to_np(inp["alpha"][s]), to_np(inp["beta"][s]), st)
        worst = max(worst, check_close(o, o_ref, "bf16", stored_bf16=True, what=f"o step {s}"))
    r = check_close(state, st, "f32", what="final state (100 steps)")
    print(f"  error/allowed: o {worst:.3f} (worst step)  state {r:.3f}", flush=True)
