"""GPU parity at the fast-forgetting end of the gate's range.

The pages give the forget gate the whole interval (0, 1) per key channel
(channel-wise fast forgetting: "Linear Attention KDA Gating in a 3:1 Hybrid
Architecture", section 2, items 3 and 5) and ask that chunk boundaries never
overflow ("Designing and Deploying Hybrid MLA and Linear Attention
Architectures", section 3).  These cases draw gates with a high mean
pre-activation (mean alpha ~0.5 or ~0.13), a quarter of the entries
log-uniform down to 1e-30 (softplus form: pre-activations up to 100) and a
few exact zeros, and compare every element with the fp64 oracle for each chunk
size, activation dtype and gate form, for the decode step and for the
chunkwise backward.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_12_amd as kda
import oracle
import synth
from tests.helpers import check_close, chunk_floor, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
ODT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _fwd_case(gate, C, act, out, mu, seed, B=2, T=300, H=2, Dk=128, Dv=128, lengths=None,
              tiny_frac=0.25, zero_frac=0.02):
    inp = synth.chunk_inputs(B, T, H, Dk, Dv, act, mu=mu, s0_std=0.05, seed=seed, device=DEV,
                             lengths=lengths)
    Tt = inp["q"].shape[1]
    g = synth.draw_strong_gate(gate, (B, Tt), H, Dk, mu, seed, DEV, tiny_frac=tiny_frac,
                               zero_frac=zero_frac)
    o, sT = kda.kda_chunk_fwd(inp["q"], inp["k"], inp["v"], g, inp["beta"],
                              initial_state=inp["initial_state"], final_state=True,
                              cu_seqlens=inp["cu_seqlens"], out_dtype=ODT[out], gate=gate,
                              chunk_size=C)
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


@pytest.mark.parametrize("C", [64, 32, 128])
@pytest.mark.parametrize("gate", ["alpha", "softplus", "scalar"])
@pytest.mark.parametrize("act,out", [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16")])
@pytest.mark.parametrize("mu", [0.0, 2.0])
def test_chunk_fwd_strong_decay(C, gate, act, out, mu):
    print(f"[chunk strong decay C={C} gate={gate} act={act} out={out} mu={mu}]", flush=True)
    _fwd_case(gate, C, act, out, mu, seed=int(101 + 10 * mu + C))


@pytest.mark.parametrize("C", [64, 32, 128])
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_chunk_fwd_strong_decay_varlen_small_heads(C, act):
    print(f"[chunk strong decay varlen C={C} act={act} d=64]", flush=True)
    _fwd_case("alpha", C, act, "f32", 1.0, seed=5, B=1, T=0, H=3, Dk=64, Dv=64,
              lengths=[1, 129, 0, 64, 17, 250])


@pytest.mark.parametrize("C", [64, 32, 128])
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_chunk_fwd_alpha_half_everywhere(C, act):
    """alpha = 0.5 on every channel and token: over a 128-token chunk the
    decay is 2^-128, past the range of a single fp32 factor 2^b or 2^-b."""
    print(f"[chunk alpha=0.5 C={C} act={act}]", flush=True)
    inp = synth.chunk_inputs(1, 384, 2, 128, 128, act, s0_std=0.05, seed=3, device=DEV)
    a = torch.full_like(inp["alpha"], 0.5)
    o, sT = kda.kda_chunk_fwd(inp["q"], inp["k"], inp["v"], a, inp["beta"],
                              initial_state=inp["initial_state"], final_state=True,
                              out_dtype=torch.float32, chunk_size=C)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.kda_fwd(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]), to_np(a),
                                  to_np(inp["beta"]), initial_state=to_np(inp["initial_state"]))
    kind = "f32" if act == "f32" else "bf16"
    r1 = check_close(o, o_ref, kind, what="o")
    r2 = check_close(sT, s_ref, kind, what="final state")
    print(f"  error/allowed: o {r1:.3f}  S_T {r2:.3f}", flush=True)


@pytest.mark.parametrize("C", [64, 32, 128])
@pytest.mark.parametrize("gate", ["alpha", "softplus", "scalar"])
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_chunk_fwd_mixed_forms(C, gate, act):
    """Mild gates everywhere except every third (sequence, chunk, head), which
    gets strong ones: the preparation kernels take the direct form for some
    chunks and list the others for the general form within one call."""
    print(f"[chunk mixed forms C={C} gate={gate} act={act}]", flush=True)
    B, T, H, D = 2, 640, 3, 128
    inp = synth.chunk_inputs(B, T, H, D, D, act, mu=-2.0, s0_std=0.05, seed=51, device=DEV)
    mild = synth.draw_gate(gate, (B, T), H, D, -2.0, 51, DEV)
    strong = synth.draw_strong_gate(gate, (B, T), H, D, 2.0, 52, DEV)
    bb = torch.arange(B, device=DEV)[:, None, None]
    cc = (torch.arange(T, device=DEV) // C)[None, :, None]
    hh = torch.arange(H, device=DEV)[None, None, :]
    sel = (bb + cc + hh) % 3 == 0
    if gate != "scalar":
        sel = sel[..., None]
    g = torch.where(sel, strong, mild).contiguous()
    o, sT = kda.kda_chunk_fwd(inp["q"], inp["k"], inp["v"], g, inp["beta"], initial_state=inp["initial_state"],
                              final_state=True, out_dtype=torch.float32, gate=gate, chunk_size=C)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.kda_fwd(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]),
                                  oracle.alpha_from_gate(to_np(g), gate, D), to_np(inp["beta"]),
                                  initial_state=to_np(inp["initial_state"]))
    kind = "f32" if act == "f32" else "bf16"
    r1 = check_close(o, o_ref, kind, what="o")
    r2 = check_close(sT, s_ref, kind, what="final state")
    print(f"  error/allowed: o {r1:.3f}  S_T {r2:.3f}", flush=True)


def test_chunk_fwd_large_keys_take_the_general_form():
    """bf16 keys and queries of norm 8 (entries above 2) with mild gates: the
    C = 64 direct form's operand check sends every chunk to the general form,
    whose factors never exceed 1; the result still matches the oracle."""
    print("[chunk large keys]", flush=True)
    inp = synth.chunk_inputs(2, 300, 2, 128, 128, "bf16", mu=-2.0, s0_std=0.05, seed=61, device=DEV)
    k = (inp["k"].float() * 8).to(torch.bfloat16)
    q = (inp["q"].float() * 8).to(torch.bfloat16)
    o, sT = kda.kda_chunk_fwd(q, k, inp["v"], inp["alpha"], inp["beta"] / 64, initial_state=inp["initial_state"],
                              final_state=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.kda_fwd(to_np(q), to_np(k), to_np(inp["v"]), to_np(inp["alpha"]), to_np(inp["beta"] / 64),
                                  initial_state=to_np(inp["initial_state"]))
    r1 = check_close(o, o_ref, "bf16", what="o")
    r2 = check_close(sT, s_ref, "bf16", what="final state")
    print(f"  error/allowed: o {r1:.3f}  S_T {r2:.3f}", flush=True)


@pytest.mark.parametrize("gate", ["alpha", "softplus", "scalar"])
@pytest.mark.parametrize("act,out", [("f32", "f32"), ("bf16", "bf16")])
def test_decode_strong_decay(gate, act, out):
    print(f"[decode strong decay gate={gate} act={act} out={out}]", flush=True)
    steps, N, H, D = 6, 4, 3, 128
    inp = synth.decode_inputs(N, H, D, D, steps, act, s0_std=0.05, seed=23, device=DEV)
    g = synth.draw_strong_gate(gate, (steps, N), H, D, 2.0, 23, DEV)
    state = inp["state"].clone()
    st_ref = to_np(inp["state"])
    for s in range(steps):
        o = kda.kda_recurrent_step(inp["q"][s], inp["k"][s], inp["v"][s], g[s], inp["beta"][s],
                                   state, out_dtype=ODT[out], gate=gate)
        torch.cuda.synchronize()
        o_ref, st_ref = oracle.kda_step(to_np(inp["q"][s]), to_np(inp["k"][s]), to_np(inp["v"][s]),
                                        oracle.alpha_from_gate(to_np(g[s]), gate, D),
                                        to_np(inp["beta"][s]), st_ref)
        check_close(o, o_ref, "f32" if out == "f32" else "bf16", stored_bf16=(out == "bf16"),
                    what=f"o step {s}")
    check_close(state, st_ref, "f32", what="state")


# ---------------------------------------------------------------------------
# Backward.  A chunk in which some channel decays below 2^-64 takes the
# general form of the backward kernels (no decay factor above 1); any other
# chunk the direct form.  The cases below reach both, alone and mixed within
# one call.  alpha = 0 exactly is outside the backward's domain (dL/dalpha
# is formed as dL/dlog(alpha) / alpha), so no entry is zeroed here.
#
# The gate gradient of the "alpha" and "scalar" forms is dL/dlog(alpha)
# divided by alpha: its absolute error is that of dL/dlog(alpha) (a reverse
# running sum over the chunk) times 1 / alpha, so at alpha << 1 it is checked
# in the log domain, alpha * dL/dalpha = dL/dlog(alpha), with the tolerance of
# every other gradient.  The "softplus" form's gradient, -sigmoid(x)
# dL/dlog(alpha), is bounded by dL/dlog(alpha) and is checked as returned.
# ---------------------------------------------------------------------------
def _bwd_strong(gate, act, g, inp, seed, lengths=None):
    B, Tt, H, Dk = inp["q"].shape
    N = B if lengths is None else len(lengths)
    up = synth.draw_upstream((B, Tt), N, H, Dk, inp["v"].shape[-1], act, 0.1, seed, DEV)
    r = kda.kda_chunk_bwd(inp["q"], inp["k"], inp["v"], g, inp["beta"], up["dout"],
                          initial_state=inp["initial_state"], dfinal_state=up["dfinal_state"],
                          cu_seqlens=inp["cu_seqlens"], gate=gate)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"]
    a = oracle.alpha_from_gate(to_np(g), gate, Dk)
    ref = oracle.kda_bwd(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]), a, to_np(inp["beta"]),
                         to_np(up["dout"]), initial_state=synth.to_f64(inp["initial_state"]),
                         dfinal_state=synth.to_f64(up["dfinal_state"]),
                         cu_seqlens=None if cu is None else cu.cpu().numpy().astype(np.int64))
    kind = "f32" if act == "f32" else "bf16"
    ratios = {}
    for name in ("dq", "dk", "dv"):
        ratios[name] = check_close(r[name], ref[name], kind, stored_bf16=(act == "bf16"), what=name)
    ratios["dbeta"] = check_close(r["dbeta"], ref["dbeta"], kind, what="dbeta")
    ratios["dS0"] = check_close(r["dinitial_state"], ref["dinitial_state"], kind, what="dS0")
    # dL/dlog(alpha) per channel and the largest running sum of its chunk
    cun = None if cu is None else cu.cpu().numpy()
    dlog = ref["dalpha"] * a
    fl = chunk_floor(dlog, cun)
    gv = to_np(g)
    if gate == "softplus":
        sig = 1.0 / (1.0 + np.exp(-gv))                  # dL/dx = -sigmoid(x) dL/dlog(alpha)
        ratios["dgate"] = check_close(r["dgate"], oracle.gate_grad(ref["dalpha"], gv, gate), kind,
                                      what="dgate", floor=sig * fl)
    elif gate == "alpha":
        ratios["dlog_gate"] = check_close(to_np(r["dgate"]) * gv, dlog, kind,
                                          what="alpha * dgate (d/dlog alpha)", floor=fl)
    else:                                                 # the channel sums of the running sums
        ratios["dlog_gate"] = check_close(to_np(r["dgate"]) * gv, dlog.sum(axis=-1), kind,
                                          what="alpha * dgate (d/dlog alpha)", floor=fl.sum(axis=-1))
    print("  error/allowed: " + "  ".join(f"{k} {v:.3f}" for k, v in ratios.items()), flush=True)


@pytest.mark.parametrize("gate", ["alpha", "softplus", "scalar"])
@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("mu", [0.0, 2.0])
def test_chunk_bwd_strong_decay(gate, act, mu):
    print(f"[bwd strong decay gate={gate} act={act} mu={mu}]", flush=True)
    seed = int(301 + 10 * mu)
    inp = synth.chunk_inputs(2, 300, 2, 128, 128, act, mu=mu, s0_std=0.05, seed=seed, device=DEV)
    g = synth.draw_strong_gate(gate, (2, 300), 2, 128, mu, seed, DEV, zero_frac=0.0)
    _bwd_strong(gate, act, g, inp, seed)


@pytest.mark.parametrize("gate", ["alpha", "softplus", "scalar"])
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_chunk_bwd_mixed_forms(gate, act):
    """Mild gates (mean alpha ~0.88) everywhere except every third
    (sequence, chunk, head), which gets strong ones: both forms of the
    backward in one call, each (chunk, head) on its own."""
    print(f"[bwd mixed forms gate={gate} act={act}]", flush=True)
    B, T, H, D = 2, 512, 3, 128
    inp = synth.chunk_inputs(B, T, H, D, D, act, mu=-2.0, s0_std=0.05, seed=41, device=DEV)
    mild = synth.draw_gate(gate, (B, T), H, D, -2.0, 41, DEV)
    strong = synth.draw_strong_gate(gate, (B, T), H, D, 2.0, 42, DEV, zero_frac=0.0)
    bb = torch.arange(B, device=DEV)[:, None, None]
    cc = (torch.arange(T, device=DEV) // 64)[None, :, None]
    hh = torch.arange(H, device=DEV)[None, None, :]
    sel = (bb + cc + hh) % 3 == 0
    if gate != "scalar":
        sel = sel[..., None]
    g = torch.where(sel, strong, mild).contiguous()
    _bwd_strong(gate, act, g, inp, 41)


@pytest.mark.parametrize("Dk,Dv", [(128, 64), (64, 128)])
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_chunk_bwd_mixed_forms_unequal_heads(Dk, Dv, act):
    """Both forms of the backward in one call where d_k != d_v: the direct
    form's preparation stages the key channels and the value columns in
    64-wide slices, so its W and U passes differ in number here."""
    print(f"[bwd mixed forms Dk={Dk} Dv={Dv} act={act}]", flush=True)
    B, T, H = 1, 384, 2
    inp = synth.chunk_inputs(B, T, H, Dk, Dv, act, mu=-2.0, s0_std=0.05, seed=43, device=DEV)
    mild = synth.draw_gate("alpha", (B, T), H, Dk, -2.0, 43, DEV)
    strong = synth.draw_strong_gate("alpha", (B, T), H, Dk, 2.0, 44, DEV, zero_frac=0.0)
    cc = (torch.arange(T, device=DEV) // 64)[None, :, None]
    hh = torch.arange(H, device=DEV)[None, None, :]
    sel = ((cc + hh) % 2 == 0)[..., None]
    g = torch.where(sel, strong, mild).contiguous()
    _bwd_strong("alpha", act, g, inp, 43)


@pytest.mark.parametrize("gate", ["alpha", "softplus"])
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_chunk_bwd_strong_decay_varlen_small_heads(gate, act):
    print(f"[bwd strong decay varlen gate={gate} act={act} d=64]", flush=True)
    lengths = [1, 129, 0, 64, 17, 250]
    inp = synth.chunk_inputs(1, 0, 3, 64, 64, act, mu=1.0, s0_std=0.05, seed=7, device=DEV, lengths=lengths)
    Tt = inp["q"].shape[1]
    g = synth.draw_strong_gate(gate, (1, Tt), 3, 64, 1.0, 7, DEV, zero_frac=0.0)
    _bwd_strong(gate, act, g, inp, 7, lengths=lengths)


@pytest.mark.parametrize("alpha", [0.5, 0.4])
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_chunk_bwd_uniform_gate_at_the_form_boundary(alpha, act):
    """alpha = 0.5 everywhere decays each channel by exactly 2^-64 over a
    64-token chunk (the direct form's limit, where 1/Gamma reaches 2^64);
    alpha = 0.4 by 2^-84.6 (the general form)."""
    print(f"[bwd uniform alpha={alpha} act={act}]", flush=True)
    inp = synth.chunk_inputs(1, 256, 2, 128, 128, act, s0_std=0.05, seed=13, device=DEV)
    g = torch.full_like(inp["alpha"], alpha)
    _bwd_strong("alpha", act, g, inp, 13)
