"""Comparison helpers shared by the parity tests.

Tolerances (stated for the fp64 oracle as reference):

* fp32 activations: norm-wise relative error  max|got - ref| / max|ref| <= 1e-4,
  and per element |got - ref| <= 1e-4 * max(|ref|, RMS(ref)), so small
  elements are held to the bound of a typical one, not only of the largest.
  (A bare element-wise relative error is ill-posed: outputs pass through zero.)
  Gate gradients are formed from dL/dlog(alpha), which the chunk form takes
  as a reverse running sum over each 64-token chunk per key channel: the
  running sums of a chunk are that chunk's own values, so an element's
  absolute error scales with the largest of them, not with the element.
  Their per-element floor therefore also takes that largest value
  (``chunk_floor``), while the norm-wise bound stays as it is.
* bf16 activations: max|got - ref| <= 2e-2 * RMS(ref) for every element of o
  (and of the final state when it is returned), RMS over the whole tensor.
  When o is stored in bf16 the stored value is additionally off by at most
  half a bf16 unit in the last place of itself (round-to-nearest of the fp32
  accumulator), so that term is added per element.  Rounding the EXACT result
  to bf16 already costs up to ~2e-2 * RMS on these distributions, so the bare
  bound cannot apply to a bf16-stored output.
"""
from __future__ import annotations

import numpy as np
import torch

BF16_REL = 2e-2
F32_NORMWISE = 1e-4


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place of |x| (0 where x == 0)."""
    ax = np.abs(x.astype(np.float64))
    out = np.zeros_like(ax)
    nz = ax > 0
    e = np.floor(np.log2(ax[nz]))
    out[nz] = np.exp2(e - 8)
    return out


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def chunk_floor(x, cu_seqlens=None, chunk: int = 64) -> np.ndarray:
    """|x| maximised over each chunk of ``chunk`` tokens and broadcast back to
    the chunk's tokens, per batch row and trailing index (head, channel).
    Chunks restart at every sequence start: with ``cu_seqlens`` (B == 1) at
    each of its offsets, otherwise at the start of each batch row."""
    a = np.abs(np.asarray(x, np.float64))
    B, T = a.shape[:2]
    out = np.zeros_like(a)
    starts = [0, T] if cu_seqlens is None else [int(c) for c in cu_seqlens]
    for b in range(B):
        for n in range(len(starts) - 1):
            for t0 in range(starts[n], starts[n + 1], chunk):
                t1 = min(t0 + chunk, starts[n + 1])
                out[b, t0:t1] = a[b, t0:t1].max(axis=0, keepdims=True)
    return out


def error_ratio(got, ref, kind: str, stored_bf16: bool = False, floor=None) -> float:
    """Error over the allowed error under the tolerance of ``kind`` ("f32" or
    "bf16"): <= 1 passes.  Non-finite values give inf.  ``floor`` (an array
    of ref's shape, fp32 only) raises each element's scale to at least it."""
    g = to_np(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {r.shape}")
    if r.size == 0:
        return 0.0
    if not np.all(np.isfinite(g)):
        return float("inf")
    err = np.abs(g - r)
    if kind == "f32":
        scale = max(np.max(np.abs(r)), 1e-30)
        rms_floor = max(float(np.sqrt(np.mean(r * r))), 1e-30)
        normwise = float(np.max(err) / scale / F32_NORMWISE)
        scale_e = np.maximum(np.abs(r), rms_floor)
        if floor is not None:
            scale_e = np.maximum(scale_e, np.asarray(floor, np.float64))
        elem = float(np.max(err / scale_e) / F32_NORMWISE)
        return max(normwise, elem)
    rms = float(np.sqrt(np.mean(r * r)))
    allow = BF16_REL * rms + (half_ulp_bf16(g) if stored_bf16 else 0.0)
    return float(np.max(err / allow))


def check_close(got, ref, kind: str, stored_bf16: bool = False, what: str = "", floor=None) -> float:
    """Assert the tolerance of ``kind`` ("f32" or "bf16"); return the error ratio
    (error / allowed, <= 1 passes)."""
    g = to_np(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    ratio = error_ratio(g, r, kind, stored_bf16, floor)
    if kind == "f32":
        assert ratio <= 1.0, (f"{what}: fp32 error {ratio * F32_NORMWISE:.3e} above {F32_NORMWISE} "
                              "(norm-wise, or element-wise with an RMS floor)")
    else:
        rms = float(np.sqrt(np.mean(r * r)))
        assert ratio <= 1.0, (f"{what}: max-abs err {np.max(np.abs(g - r)):.3e} vs 2e-2*RMS={BF16_REL*rms:.3e}"
                              f" (ratio {ratio:.3f}, stored_bf16={stored_bf16})")
    return ratio
