"""Independence of (sequence, head) pairs, checked with a poisoned input.

Sequences and heads never mix in the layer: every (sequence, head) keeps its
own memory S, and the chunked form only reorganises the work inside one
sequence ("Hybrid Linear Attention Architectures...", Hardware-Aware Chunkwise
Parallelism: the state is passed from chunk to chunk of the same sequence).
A NaN placed in one token of one (sequence, head) must therefore leave every
output of every other pair bit-identical to a clean run, and also every chunk
of the poisoned pair that ends before the poisoned token.
"""
import pytest
import torch

import gated_delta_rule_12_amd as kda
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _poison(t, idx):
    x = t.clone()
    x[idx] = float("nan")
    return x


def _bits(t):
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[t.element_size()])


def _same_except(a, b, mask_fn, what):
    """a and b bit-identical wherever mask_fn(shape-like bool tensor) is False."""
    diff = _bits(a) != _bits(b)
    keep = ~mask_fn(diff)
    assert not torch.any(diff & keep), f"{what}: a poisoned input changed another (sequence, head)"


@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("which", ["v", "k", "alpha"])
@pytest.mark.parametrize("varlen", [False, True])
def test_chunk_fwd_nan_stays_in_its_pair(act, which, varlen):
    print(f"[nan isolation chunk act={act} poison={which} varlen={varlen}]", flush=True)
    if varlen:
        inp = synth.chunk_inputs(1, 0, 4, 128, 128, act, s0_std=0.05, seed=17, device=DEV,
                                 lengths=[130, 300, 0, 77, 200])
        n_bad, t_bad, h_bad = 1, 130 + 150, 2          # sequence 1, its token 150
        seq_of_row = torch.repeat_interleave(torch.arange(5, device=DEV),
                                             torch.tensor([130, 300, 0, 77, 200], device=DEV))
        b_idx = (0, t_bad, h_bad)
        first_row = 130
    else:
        inp = synth.chunk_inputs(3, 300, 4, 128, 128, act, s0_std=0.05, seed=17, device=DEV)
        n_bad, t_bad, h_bad = 1, 150, 2
        b_idx = (n_bad, t_bad, h_bad)
        first_row = 0
    args = dict(initial_state=inp["initial_state"], final_state=True, cu_seqlens=inp["cu_seqlens"],
                out_dtype=torch.float32)
    o0, s0 = kda.kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], **args)
    bad = dict(inp)
    bad[which] = _poison(inp[which], b_idx)
    o1, s1 = kda.kda_chunk_fwd(bad["q"], bad["k"], bad["v"], bad["alpha"], bad["beta"], **args)
    torch.cuda.synchronize()
    chunk_start = first_row + (t_bad - first_row) // 64 * 64

    def o_mask(d):
        m = torch.zeros_like(d)
        if varlen:
            rows = (seq_of_row == n_bad) & (torch.arange(d.shape[1], device=DEV) >= chunk_start)
            m[0, rows, h_bad] = True
        else:
            m[n_bad, chunk_start:, h_bad] = True
        return m

    def s_mask(d):
        m = torch.zeros_like(d)
        m[n_bad, h_bad] = True
        return m

    _same_except(o0, o1, o_mask, "o")
    _same_except(s0, s1, s_mask, "final state")
    assert torch.isnan(s1[n_bad, h_bad]).any(), "the poisoned pair should carry the NaN"


def test_decode_nan_stays_in_its_pair():
    print("[nan isolation decode]", flush=True)
    inp = synth.decode_inputs(6, 4, 128, 128, 2, "bf16", s0_std=0.05, seed=29, device=DEV)
    st0 = inp["state"].clone()
    st1 = inp["state"].clone()
    for s in range(2):
        k = inp["k"][s]
        o0 = kda.kda_recurrent_step(inp["q"][s], k, inp["v"][s], inp["alpha"][s], inp["beta"][s], st0,
                                    out_dtype=torch.float32)
        kb = _poison(k, (3, 1, 5)) if s == 0 else k
        o1 = kda.kda_recurrent_step(inp["q"][s], kb, inp["v"][s], inp["alpha"][s], inp["beta"][s], st1,
                                    out_dtype=torch.float32)
        torch.cuda.synchronize()

        def pair_mask(d):
            m = torch.zeros_like(d)
            m[3, 1] = True
            return m
        _same_except(o0, o1, pair_mask, f"o step {s}")
        _same_except(st0, st1, pair_mask, f"state step {s}")
    assert torch.isnan(st1[3, 1]).any()


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_chunk_bwd_nan_stays_in_its_pair(act):
    print(f"[nan isolation backward act={act}]", flush=True)
    B, T, H, D = 3, 200, 4, 128
    inp = synth.chunk_inputs(B, T, H, D, D, act, s0_std=0.05, seed=37, device=DEV)
    up = synth.draw_upstream((B, T), B, H, D, D, act, 0.1, 37, DEV)
    args = dict(initial_state=inp["initial_state"], dfinal_state=up["dfinal_state"])
    r0 = kda.kda_chunk_bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], up["dout"], **args)
    dbad = _poison(up["dout"], (1, 120, 2))
    r1 = kda.kda_chunk_bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], dbad, **args)
    torch.cuda.synchronize()

    def tok_mask(d):
        m = torch.zeros_like(d, dtype=torch.bool)
        m[1, :, 2] = True
        return m

    def st_mask(d):
        m = torch.zeros_like(d, dtype=torch.bool)
        m[1, 2] = True
        return m
    for key in ("dq", "dk", "dv", "dgate", "dbeta"):
        _same_except(r0[key], r1[key], tok_mask, key)
    _same_except(r0["dinitial_state"], r1["dinitial_state"], st_mask, "dinitial_state")
    assert torch.isnan(r1["dinitial_state"][1, 2]).any()
