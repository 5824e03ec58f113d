"""Comparison helpers shared by the parity tests.

Tolerances (stated for the fp64 oracle as reference):

* fp32 activations: norm-wise relative error  max|got - ref| / max|ref| <= 1e-4,
  and per element |got - ref| <= 1e-4 * max(|ref|, RMS(ref)), so small
  elements are held to the bound of a typical one, not only of the largest.
  (A bare element-wise relative error is ill-posed: outputs pass through zero.)
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


def error_ratio(got, ref, kind: str, stored_bf16: bool = False) -> float:
    """Error over the allowed error under the tolerance of ``kind`` ("f32" or
    "bf16"): <= 1 passes.  Non-finite values give inf."""
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
        floor = max(float(np.sqrt(np.mean(r * r))), 1e-30)
        normwise = float(np.max(err) / scale / F32_NORMWISE)
        elem = float(np.max(err / np.maximum(np.abs(r), floor)) / F32_NORMWISE)
        return max(normwise, elem)
    rms = float(np.sqrt(np.mean(r * r)))
    allow = BF16_REL * rms + (half_ulp_bf16(g) if stored_bf16 else 0.0)
    return float(np.max(err / allow))


def check_close(got, ref, kind: str, stored_bf16: bool = False, what: str = "") -> float:
    """Assert the tolerance of ``kind`` ("f32" or "bf16"); return the error ratio
    (error / allowed, <= 1 passes)."""
    g = to_np(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    ratio = error_ratio(g, r, kind, stored_bf16)
    if kind == "f32":
        assert ratio <= 1.0, (f"{what}: fp32 error {ratio * F32_NORMWISE:.3e} above {F32_NORMWISE} "
                              "(norm-wise, or element-wise with an RMS floor)")
    else:
        rms = float(np.sqrt(np.mean(r * r)))
        assert ratio <= 1.0, (f"{what}: max-abs err {np.max(np.abs(g - r)):.3e} vs 2e-2*RMS={BF16_REL*rms:.3e}"
                              f" (ratio {ratio:.3f}, stored_bf16={stored_bf16})")
    return ratio
