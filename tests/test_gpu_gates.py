"""GPU parity of the other forget-gate forms (gate="softplus": bf16
pre-activation x with log alpha = -softplus(x); gate="scalar": one fp32 alpha
per token and head) against the fp64 oracle, through the *_gated C entry
points.  The oracle receives the alpha each form stands for
(oracle.alpha_from_gate), computed in fp64 from the exact device values."""
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
GATES = ["softplus", "scalar"]


def _chunk_case(gate, B, T, H, Dk, Dv, act, out, seed, lengths=None, s0_std=0.02, mu=-2.0):
    inp = synth.chunk_inputs(B, T, H, Dk, Dv, act, mu=mu, s0_std=s0_std, seed=seed, device=DEV,
                             lengths=lengths)
    Tt = inp["q"].shape[1]
    g = synth.draw_gate(gate, (B, Tt), H, Dk, mu, seed, DEV)
    o, sT = kda.kda_chunk_fwd(inp["q"], inp["k"], inp["v"], g, inp["beta"],
                              initial_state=inp["initial_state"], final_state=True,
                              cu_seqlens=inp["cu_seqlens"], out_dtype=ODT[out], gate=gate)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"]
    o_ref, s_ref = oracle.kda_fwd(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]),
                                  oracle.alpha_from_gate(to_np(g), gate, Dk), to_np(inp["beta"]),
                                  initial_state=synth.to_f64(inp["initial_state"]),
                                  cu_seqlens=None if cu is None else cu.cpu().numpy().astype(np.int64))
    kind = "f32" if act == "f32" else "bf16"
    r1 = check_close(o, o_ref, kind, stored_bf16=(out == "bf16"), what="o")
    r2 = check_close(sT, s_ref, kind, what="final state")
    print(f"  error/allowed: o {r1:.3f}  S_T {r2:.3f}", flush=True)


@pytest.mark.parametrize("gate", GATES)
@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 64), (64, 128)])
@pytest.mark.parametrize("act,out", [("f32", "f32"), ("bf16", "bf16")])
@pytest.mark.parametrize("T", [64, 200])
def test_chunk_gate_small(gate, Dk, Dv, act, out, T):
    print(f"[chunk gate={gate} Dk={Dk} Dv={Dv} act={act} out={out} T={T}]", flush=True)
    _chunk_case(gate, 2, T, 3, Dk, Dv, act, out, seed=31 + T)


@pytest.mark.parametrize("gate", GATES)
def test_chunk_gate_varlen(gate):
    print(f"[chunk gate={gate} varlen]", flush=True)
    _chunk_case(gate, 1, 0, 4, 128, 128, "bf16", "bf16", seed=7, lengths=[0, 70, 1, 256, 133])


@pytest.mark.parametrize("gate", GATES)
def test_chunk_gate_medium(gate):
    """B=2, H=8, T=4096, d=128, bf16 (the shape of the element-wise workload)."""
    print(f"[chunk gate={gate} B2 H8 T4096 d128 bf16]", flush=True)
    _chunk_case(gate, 2, 4096, 8, 128, 128, "bf16", "f32", seed=1, s0_std=None)


@pytest.mark.parametrize("gate", GATES)
@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 64)])
@pytest.mark.parametrize("act,out", [("f32", "f32"), ("bf16", "bf16")])
def test_decode_gate_steps(gate, Dk, Dv, act, out):
    print(f"[decode gate={gate} Dk={Dk} Dv={Dv} act={act} out={out}]", flush=True)
    steps, N, H = 5, 4, 3
    inp = synth.decode_inputs(N, H, Dk, Dv, steps, act, mu=-2.0, s0_std=0.02, seed=19, device=DEV)
    g = synth.draw_gate(gate, (steps, N), H, Dk, -2.0, 19, DEV)
    state = inp["state"].clone()
    st_ref = to_np(inp["state"])
    for s in range(steps):
        o = kda.kda_recurrent_step(inp["q"][s], inp["k"][s], inp["v"][s], g[s], inp["beta"][s],
                                   state, out_dtype=ODT[out], gate=gate)
        torch.cuda.synchronize()
        o_ref, st_ref = oracle.kda_step(to_np(inp["q"][s]), to_np(inp["k"][s]), to_np(inp["v"][s]),
                                        oracle.alpha_from_gate(to_np(g[s]), gate, Dk),
                                        to_np(inp["beta"][s]), st_ref)
        if out == "f32":
            check_close(o, o_ref, "f32", what=f"o step {s}")
        else:
            check_close(o, o_ref, "bf16", stored_bf16=True, what=f"o step {s}")
    check_close(state, st_ref, "f32", what="state")
