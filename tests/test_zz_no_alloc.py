"""The allocation-free forward (kda_chunk_fwd_static) against the workspace
forward (kda_chunk_fwd_gated), through the C ABI: two calls in a row, the
second on a smaller, packed problem, each bit-identical to the workspace
entry point on the same inputs and within the fp64 oracle's tolerance."""
import numpy as np
import pytest
import torch

import gated_delta_rule_12_amd as kda
import oracle
import synth
from tests.helpers import check_close, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run_pair(inp, gate_name, g, out_dtype):
    args = dict(initial_state=inp["initial_state"], cu_seqlens=inp["cu_seqlens"], out_dtype=out_dtype,
                gate=gate_name)
    o_ws, s_ws = kda.kda_chunk_fwd(inp["q"], inp["k"], inp["v"], g, inp["beta"], final_state=True, **args)
    o_st, s_st = kda.kda_chunk_fwd_static(inp["q"], inp["k"], inp["v"], g, inp["beta"], final_state=True,
                                          **args)
    torch.cuda.synchronize()
    return o_ws, s_ws, o_st, s_st


def _check_vs_oracle(inp, g, gate_name, o, sT, kind, stored_bf16):
    cu = inp["cu_seqlens"]
    Dk = inp["q"].shape[-1]
    o_ref, s_ref = oracle.kda_fwd(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]),
                                  oracle.alpha_from_gate(to_np(g), gate_name, Dk), to_np(inp["beta"]),
                                  initial_state=synth.to_f64(inp["initial_state"]),
                                  cu_seqlens=None if cu is None else cu.cpu().numpy().astype(np.int64))
    r1 = check_close(o, o_ref, kind, stored_bf16=stored_bf16, what="o (static workspace)")
    r2 = check_close(sT, s_ref, kind, what="final state (static workspace)")
    print(f"  error/allowed: o {r1:.3f}  S_T {r2:.3f}", flush=True)


def test_static_workspace_matches_workspace_entry_point():
    # first call: B=2, T=1000, H=8, d=128, bf16 (256 chunk-heads, ~18 MiB of workspace)
    print("[static workspace, call 1: B2 T1000 H8 d128 bf16]", flush=True)
    inp = synth.chunk_inputs(2, 1000, 8, 128, 128, "bf16", s0_std=0.05, seed=71, device=DEV)
    need = kda.kda_chunk_fwd_workspace_bytes(2, 1000, 8, 128, 128, False, 0, 64, torch.bfloat16)
    assert 16 << 20 < need <= kda.KDA_STATIC_WORKSPACE_BYTES
    o_ws, s_ws, o_st, s_st = _run_pair(inp, "alpha", inp["alpha"], torch.bfloat16)
    assert torch.equal(o_ws, o_st) and torch.equal(s_ws, s_st)
    _check_vs_oracle(inp, inp["alpha"], "alpha", o_st, s_st, "bf16", True)

    # second call, smaller: 3 packed sequences, 4 heads, d=64, fp32, softplus gate
    print("[static workspace, call 2: packed, H4 d64 f32 softplus]", flush=True)
    inp2 = synth.chunk_inputs(1, 0, 4, 64, 64, "f32", s0_std=0.05, seed=72, device=DEV,
                              lengths=[100, 0, 333])
    g2 = synth.draw_gate("softplus", (1, 433), 4, 64, -2.0, 72, DEV)
    o_ws, s_ws, o_st, s_st = _run_pair(inp2, "softplus", g2, torch.float32)
    assert torch.equal(o_ws, o_st) and torch.equal(s_ws, s_st)
    _check_vs_oracle(inp2, g2, "softplus", o_st, s_st, "f32", False)


def test_static_workspace_rejects_oversized_problem():
    print("[static workspace, oversized]", flush=True)
    inp = synth.chunk_inputs(1, 4096, 32, 128, 128, "bf16", seed=73, device=DEV)
    with pytest.raises(kda.KDAError) as e:
        kda.kda_chunk_fwd_static(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"])
    assert e.value.status == kda.KDA_ERROR_WORKSPACE_TOO_SMALL
