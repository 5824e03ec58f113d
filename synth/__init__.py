"""Seeded synthetic inputs for the KDA layer.

This module only draws random numbers in the shapes and value distributions
of the workloads; it holds none of the layer's arithmetic, and both the HIP
path's callers and the oracle's callers take their inputs from here.

Value recipe (the same for every workload unless a field overrides it):
  q, k  ~ N(0, 1), L2-normalised per (token, head), then cast to the
          activation dtype (round-to-nearest-even)
  v     ~ N(0, 1), cast to the activation dtype
  beta  = sigmoid(N(0, 1)) per (token, head), fp32
  alpha = exp(-softplus(N(mu, 1))) per (token, head, key channel), fp32
  S_0   = N(0, s0_std) fp32 per (sequence, head), or absent

Upstream gradients of a backward (``draw_upstream``): dO ~ N(0, 1) cast to
the activation dtype, dS_T ~ N(0, ds_std) fp32 per (sequence, head), or absent.

Other gate forms (``draw_gate``): "softplus" passes the pre-activation
x = N(mu, 1) itself, cast to bf16; "scalar" draws one
alpha = exp(-softplus(N(mu, 1))) per (token, head), fp32.

Every tensor is drawn from a torch.Generator seeded from (seed, tensor tag),
on the device where it is generated; a run is reproducible on the same
device type.  The oracle receives the exact values the GPU receives (they are
copied to the host), never a regenerated approximation.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch
import torch.nn.functional as F

_TAGS = {"q": 1, "k": 2, "v": 3, "beta": 4, "alpha": 5, "s0": 6, "len": 7, "gx": 8, "ga": 9,
         "do": 10, "dst": 11, "sg": 12}


def _gen(seed: int, tag: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1000003 + _TAGS[tag] * 7919) & 0x7FFFFFFFFFFFFFFF)
    return g


def _act_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


@dataclass
class Workload:
    """A named workload shape.  ``kind`` is "chunk", "varlen" or "decode"."""
    name: str
    kind: str
    H: int
    Dk: int
    Dv: int
    dtype: str = "bf16"
    mu: float = -2.0
    s0_std: Optional[float] = None
    B: int = 1
    T: int = 0
    chunk_size: int = 64
    num_seqs: int = 0
    len_lo: int = 0
    len_hi: int = 0
    steps: int = 0
    extra: dict = field(default_factory=dict)


# The five workloads of the benchmark plan, by index.
WORKLOADS = {
    0: Workload("kda_fwd_B1_H1_T256_d64_f32", "chunk", H=1, Dk=64, Dv=64, dtype="f32",
                mu=-2.0, s0_std=None, B=1, T=256),
    1: Workload("kda_chunk_fwd_B2_H8_T4096_d128_bf16", "chunk", H=8, Dk=128, Dv=128,
                dtype="bf16", mu=-2.0, s0_std=None, B=2, T=4096),
    2: Workload("kda_chunk_fwd_B1_H32_T65536_d128_bf16", "chunk", H=32, Dk=128, Dv=128,
                dtype="bf16", mu=-3.0, s0_std=0.02, B=1, T=65536),
    3: Workload("kda_decode_N256_H32_d128_bf16_100steps", "decode", H=32, Dk=128, Dv=128,
                dtype="bf16", mu=-2.0, s0_std=0.02, B=256, steps=100),
    4: Workload("kda_varlen_N64_len512to32768_H16_d128_bf16", "varlen", H=16, Dk=128, Dv=128,
                dtype="bf16", mu=-2.0, s0_std=0.02, num_seqs=64, len_lo=512, len_hi=32768),
}


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-30)


def draw_qkv_gates(lead: tuple, H: int, Dk: int, Dv: int, dtype: str, mu: float,
                   seed: int, device) -> dict:
    """q, k, v, alpha, beta with leading shape ``lead`` (e.g. (B, T) or (N,))."""
    act = _act_dtype(dtype)
    shp_k = tuple(lead) + (H, Dk)
    shp_v = tuple(lead) + (H, Dv)
    q = _unit_rows(torch.randn(shp_k, generator=_gen(seed, "q", device), device=device)).to(act)
    k = _unit_rows(torch.randn(shp_k, generator=_gen(seed, "k", device), device=device)).to(act)
    v = torch.randn(shp_v, generator=_gen(seed, "v", device), device=device).to(act)
    beta = torch.sigmoid(torch.randn(tuple(lead) + (H,), generator=_gen(seed, "beta", device),
                                     device=device))
    x = torch.randn(shp_k, generator=_gen(seed, "alpha", device), device=device) + mu
    alpha = torch.exp(-F.softplus(x))
    return dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(),
                alpha=alpha.contiguous(), beta=beta.contiguous())


def draw_gate(kind: str, lead: tuple, H: int, Dk: int, mu: float, seed: int, device):
    """The forget gate in one of the forms of the library's ``gate=`` argument:
    "alpha" (fp32 [lead, H, Dk]), "softplus" (bf16 pre-activation
    [lead, H, Dk]) or "scalar" (fp32 alpha [lead, H])."""
    if kind == "alpha":
        x = torch.randn(tuple(lead) + (H, Dk), generator=_gen(seed, "alpha", device), device=device) + mu
        return torch.exp(-F.softplus(x)).contiguous()
    if kind == "softplus":
        x = torch.randn(tuple(lead) + (H, Dk), generator=_gen(seed, "gx", device), device=device) + mu
        return x.to(torch.bfloat16).contiguous()
    if kind == "scalar":
        x = torch.randn(tuple(lead) + (H,), generator=_gen(seed, "ga", device), device=device) + mu
        return torch.exp(-F.softplus(x)).contiguous()
    raise ValueError(kind)


def draw_strong_gate(kind: str, lead: tuple, H: int, Dk: int, mu: float, seed: int, device,
                     tiny_frac: float = 0.25, tiny_lo: float = 1e-30, zero_frac: float = 0.02):
    """A forget gate that reaches the fast-forgetting end of its range.

    As ``draw_gate`` with mean pre-activation ``mu``, then a random
    ``tiny_frac`` of the entries is replaced by alpha ~ log-uniform on
    [tiny_lo, 1e-3] and a random ``zero_frac`` by alpha = 0 exactly ("alpha"
    and "scalar" forms).  For "softplus" the replaced entries take the
    pre-activation x ~ U[7, 100] (alpha = 1 / (1 + e^x) from 1e-3 down to
    4e-44), and no entry is exactly 0.
    """
    g = draw_gate(kind, lead, H, Dk, mu, seed, device)
    gen = _gen(seed, "sg", device)
    u = torch.rand(g.shape, generator=gen, device=device)
    w = torch.rand(g.shape, generator=gen, device=device)
    tiny = u < tiny_frac
    if kind == "softplus":
        x = (7.0 + 93.0 * w).to(torch.bfloat16)
        return torch.where(tiny, x, g).contiguous()
    lo, hi = torch.log(torch.tensor(tiny_lo)), torch.log(torch.tensor(1e-3))
    a = torch.exp(lo + (hi - lo) * w)
    g = torch.where(tiny, a, g)
    g = torch.where((u >= tiny_frac) & (u < tiny_frac + zero_frac), torch.zeros_like(g), g)
    return g.contiguous()


def draw_upstream(lead: tuple, N: int, H: int, Dk: int, Dv: int, dtype: str,
                  ds_std: Optional[float], seed: int, device) -> dict:
    """Upstream gradients of a backward: dout [lead, H, Dv] in the activation
    dtype and dfinal_state [N, H, Dk, Dv] fp32 (None when ds_std is None)."""
    do = torch.randn(tuple(lead) + (H, Dv), generator=_gen(seed, "do", device), device=device)
    ds = None
    if ds_std is not None:
        ds = torch.randn((N, H, Dk, Dv), generator=_gen(seed, "dst", device), device=device) * ds_std
    return {"dout": do.to(_act_dtype(dtype)).contiguous(), "dfinal_state": ds}


def draw_state(N: int, H: int, Dk: int, Dv: int, std: Optional[float], seed: int, device):
    if std is None:
        return None
    return torch.randn((N, H, Dk, Dv), generator=_gen(seed, "s0", device), device=device) * std


def varlen_lengths(num_seqs: int, lo: int, hi: int, seed: int) -> list:
    """Sequence lengths ~ Uniform{lo..hi}, drawn on the host."""
    g = _gen(seed, "len", "cpu")
    return [int(x) for x in torch.randint(lo, hi + 1, (num_seqs,), generator=g)]


def cu_from_lengths(lengths) -> torch.Tensor:
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def chunk_inputs(B: int, T: int, H: int, Dk: int, Dv: int, dtype: str = "bf16",
                 mu: float = -2.0, s0_std: Optional[float] = None, seed: int = 0,
                 device="cpu", lengths=None) -> dict:
    """Inputs of one chunked forward.  With ``lengths`` the batch is packed:
    B must be 1, T = sum(lengths), and ``cu_seqlens`` (int32) is returned."""
    out = {}
    if lengths is not None:
        if B != 1:
            raise ValueError("packed inputs need B == 1")
        cu = cu_from_lengths(lengths)
        T = int(cu[-1])
        out["cu_seqlens"] = cu.to(device)
        N = len(lengths)
    else:
        out["cu_seqlens"] = None
        N = B
    out.update(draw_qkv_gates((B, T), H, Dk, Dv, dtype, mu, seed, device))
    out["initial_state"] = draw_state(N, H, Dk, Dv, s0_std, seed, device)
    return out


def decode_inputs(N: int, H: int, Dk: int, Dv: int, steps: int, dtype: str = "bf16",
                  mu: float = -2.0, s0_std: Optional[float] = 0.02, seed: int = 0,
                  device="cpu") -> dict:
    """Per-step q, k, v, alpha, beta with leading shape (steps, N) plus the
    starting state [N, H, Dk, Dv]."""
    out = draw_qkv_gates((steps, N), H, Dk, Dv, dtype, mu, seed, device)
    st = draw_state(N, H, Dk, Dv, s0_std, seed, device)
    if st is None:
        st = torch.zeros((N, H, Dk, Dv), device=device)
    out["state"] = st
    return out


def workload_inputs(idx: int, device="cpu", seed: Optional[int] = None) -> dict:
    """Inputs of workload ``idx`` at full size, generated on ``device``."""
    w = WORKLOADS[idx]
    s = idx if seed is None else seed
    if w.kind == "chunk":
        return chunk_inputs(w.B, w.T, w.H, w.Dk, w.Dv, w.dtype, w.mu, w.s0_std, s, device)
    if w.kind == "varlen":
        lens = varlen_lengths(w.num_seqs, w.len_lo, w.len_hi, s)
        return chunk_inputs(1, 0, w.H, w.Dk, w.Dv, w.dtype, w.mu, w.s0_std, s, device,
                            lengths=lens)
    if w.kind == "decode":
        return decode_inputs(w.B, w.H, w.Dk, w.Dv, w.steps, w.dtype, w.mu, w.s0_std, s, device)
    raise ValueError(w.kind)


def to_f64(x: Optional[torch.Tensor]):
    """Exact host float64 copy (numpy) of a tensor, or None."""
    if x is None:
        return None
    return x.detach().to("cpu").to(torch.float64).numpy()
