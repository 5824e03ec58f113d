"""GPU parity of the chunkwise backward (kda_chunk_bwd, through the C ABI)
against the fp64 oracle's backward of the token recurrence (oracle.kda_bwd,
with oracle.gate_grad for the gate forms), on the exact device inputs.

Tolerances as for the forward (tests/helpers.py): fp32 activations,
norm-wise 1e-4 per gradient tensor; bf16 activations, max-abs 2e-2 x RMS of
the oracle's tensor, plus half a bf16 ulp for the gradients stored in bf16
(dq, dk, dv)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_12_amd as kda
import oracle
import synth
from tests.helpers import check_close, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bwd_case(B, T, H, Dk, Dv, act, seed, gate="alpha", lengths=None, s0_std=0.05, ds_std=1.0,
              need_ds0=True, mu=-2.0):
    inp = synth.chunk_inputs(B, T, H, Dk, Dv, act, mu=mu, s0_std=s0_std, seed=seed, device=DEV,
                             lengths=lengths)
    Tt = inp["q"].shape[1]
    N = B if lengths is None else len(lengths)
    g = inp["alpha"] if gate == "alpha" else synth.draw_gate(gate, (B, Tt), H, Dk, mu, seed, DEV)
    up = synth.draw_upstream((B, Tt), N, H, Dk, Dv, act, ds_std, seed, DEV)
    r = kda.kda_chunk_bwd(inp["q"], inp["k"], inp["v"], g, inp["beta"], up["dout"],
                          initial_state=inp["initial_state"], dfinal_state=up["dfinal_state"],
                          cu_seqlens=inp["cu_seqlens"], need_dinitial_state=need_ds0, gate=gate)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"]
    ref = oracle.kda_bwd(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]),
                         oracle.alpha_from_gate(to_np(g), gate, Dk), to_np(inp["beta"]),
                         to_np(up["dout"]), initial_state=synth.to_f64(inp["initial_state"]),
                         dfinal_state=synth.to_f64(up["dfinal_state"]),
                         cu_seqlens=None if cu is None else cu.cpu().numpy().astype(np.int64))
    ref["dgate"] = oracle.gate_grad(ref["dalpha"], to_np(g), gate)
    kind = "f32" if act == "f32" else "bf16"
    ratios = {}
    for name in ("dq", "dk", "dv"):
        ratios[name] = check_close(r[name], ref[name], kind, stored_bf16=(act == "bf16"), what=name)
    for name in ("dgate", "dbeta"):
        ratios[name] = check_close(r[name], ref[name], kind, what=name)
    if need_ds0:
        ratios["dS0"] = check_close(r["dinitial_state"], ref["dinitial_state"], kind, what="dS0")
    else:
        assert r["dinitial_state"] is None
    print("  error/allowed: " + "  ".join(f"{k} {v:.3f}" for k, v in ratios.items()), flush=True)
    return ratios


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("T", [64, 200])
def test_bwd_small(Dk, Dv, act, T):
    print(f"[bwd Dk={Dk} Dv={Dv} act={act} T={T}]", flush=True)
    _bwd_case(2, T, 2, Dk, Dv, act, seed=101 + T)


@pytest.mark.parametrize("gate", ["softplus", "scalar"])
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_bwd_gate_forms(gate, act):
    print(f"[bwd gate={gate} act={act}]", flush=True)
    _bwd_case(2, 200, 2, 128, 128, act, seed=211, gate=gate)


@pytest.mark.parametrize("gate", ["alpha", "softplus", "scalar"])
def test_bwd_varlen(gate):
    """Packed sequences with an empty and a one-token sequence; chunks restart
    at every sequence start."""
    print(f"[bwd varlen gate={gate}]", flush=True)
    _bwd_case(1, 0, 3, 128, 128, "bf16", seed=5, gate=gate, lengths=[0, 70, 1, 256, 133])


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_bwd_chunk_counts_past_the_unrolled_rounds(act):
    """Sequences of 5, 6 and 3 chunks (ragged tails): the state passes run
    their operand rings in whole rounds of three (checkpoint) or two
    (reverse) chunks plus a remainder, and these lengths reach every
    remainder after at least one whole round."""
    print(f"[bwd chunk counts act={act}]", flush=True)
    _bwd_case(1, 0, 2, 128, 128, act, seed=31, lengths=[300, 327, 129])


def test_bwd_without_state_arguments():
    print("[bwd no S0, no dS_T, no dS0]", flush=True)
    _bwd_case(2, 130, 2, 128, 128, "f32", seed=17, s0_std=None, ds_std=None, need_ds0=False)
    _bwd_case(2, 130, 2, 64, 64, "bf16", seed=18, s0_std=None, ds_std=None, need_ds0=True)


def test_bwd_zero_length_sequences_pass_state_gradient():
    """All sequences empty except one: dS_0 = dS_T where nothing happens."""
    print("[bwd empty sequences]", flush=True)
    _bwd_case(1, 0, 2, 64, 64, "f32", seed=23, lengths=[0, 0, 65, 0])


def test_bwd_medium():
    """B=2, H=8, T=4096, d=128, bf16 (the shape of the element-wise workload)."""
    print("[bwd B2 H8 T4096 d128 bf16]", flush=True)
    _bwd_case(2, 4096, 8, 128, 128, "bf16", seed=1, s0_std=None, ds_std=1.0)


def test_bwd_repeatable():
    """Two calls on the same inputs give bit-identical gradients (no atomics
    on the paths whose order could vary)."""
    inp = synth.chunk_inputs(1, 300, 2, 128, 128, "bf16", s0_std=0.05, seed=3, device=DEV)
    up = synth.draw_upstream((1, 300), 1, 2, 128, 128, "bf16", 1.0, 3, DEV)
    args = (inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], up["dout"])
    r1 = kda.kda_chunk_bwd(*args, initial_state=inp["initial_state"], dfinal_state=up["dfinal_state"])
    r2 = kda.kda_chunk_bwd(*args, initial_state=inp["initial_state"], dfinal_state=up["dfinal_state"])
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "dgate", "dbeta", "dinitial_state"):
        assert torch.equal(r1[name], r2[name]), name


def test_bwd_workload2_full():
    """B=1, H=32, T=65536, d=128, slow decay, random S0: the backward the
    benchmark times (same inputs, dO and dS_T ~ N(0, 1)), every element of
    every gradient against the oracle's backward on all 32 heads."""
    w = synth.WORKLOADS[2]
    print(f"[bwd {w.name}]", flush=True)
    inp = synth.workload_inputs(2, device=DEV)
    up = synth.draw_upstream((w.B, w.T), w.B, w.H, w.Dk, w.Dv, w.dtype, 1.0, 2, DEV)
    r = kda.kda_chunk_bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], up["dout"],
                          initial_state=inp["initial_state"], dfinal_state=up["dfinal_state"])
    torch.cuda.synchronize()
    ref = oracle.kda_bwd(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]), to_np(inp["alpha"]),
                         to_np(inp["beta"]), to_np(up["dout"]), initial_state=to_np(inp["initial_state"]),
                         dfinal_state=to_np(up["dfinal_state"]))
    ratios = {}
    for name in ("dq", "dk", "dv", "dalpha", "dbeta"):
        got = r["dgate" if name == "dalpha" else name]
        ratios[name] = check_close(got, ref[name], "bf16", stored_bf16=name in ("dq", "dk", "dv"), what=name)
        del got
    ratios["dS0"] = check_close(r["dinitial_state"], ref["dinitial_state"], "bf16", what="dS0")
    print("  error/allowed: " + "  ".join(f"{k} {v:.3f}" for k, v in ratios.items()), flush=True)
