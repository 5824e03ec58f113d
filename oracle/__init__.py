"""KDA fp64 CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP product path never imports,
links or calls it, and the two share no code.

Two implementations of the same mathematics live here:

* ``kda_fwd`` / ``kda_step`` -- the token-by-token recurrence in double
  precision (``kda_oracle.c``), the plain definition of what the layer
  computes ("Hybrid Linear Attention Architectures...", "Core Module Design",
  Stage 3; "Linear Attention KDA Gating in a 3:1 Hybrid Architecture",
  section 2, item 5).
* ``kda_bwd`` -- reverse-mode differentiation of that recurrence, token by
  token (the vector-Jacobian product of a training backward), and
  ``gate_grad`` for the chain rule from alpha to the other gate forms.
* ``oracle.chunked`` -- the chunkwise form of "Linear Attention KDA Gating in
  a 3:1 Hybrid Architecture", sections 3.1 and 3.2, in numpy fp64, exposing
  its per-chunk intermediates.  It is pinned to the recurrence by the tests.

Inputs are numpy arrays; they are converted to float64 (exactly, for fp32 or
bf16-valued data) before the call.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
SRC_PATH = os.path.join(_HERE, "kda_oracle.c")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libkda_oracle.so``."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fPIC", "-shared", "-pthread",
               "-Wall", "-Wextra", "-o", tmp, SRC_PATH]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lp = ctypes.POINTER(ctypes.c_int64)
        ip = ctypes.POINTER(ctypes.c_int)
        lib.kda_oracle_fwd.restype = ctypes.c_int
        lib.kda_oracle_fwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, lp, ctypes.c_int, dp,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ip]
        lib.kda_oracle_bwd.restype = ctypes.c_int
        lib.kda_oracle_bwd.argtypes = [dp, dp, dp, dp, dp, dp, lp, ctypes.c_int, dp, dp,
                                       dp, dp, dp, dp, dp, dp, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ip]
        lib.kda_oracle_step.restype = ctypes.c_int
        lib.kda_oracle_step.argtypes = [dp, dp, dp, dp, dp, dp, dp, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ip]
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def alpha_from_gate(gate, kind: str, Dk: int):
    """The per-channel forget gate alpha (fp64) that a gate given in the form
    ``kind`` stands for:

    * "alpha"    -- alpha itself, [..., Dk].
    * "softplus" -- the pre-activation x, [..., Dk]: log alpha = -softplus(x),
      softplus(x) = log(1 + e^x), evaluated as logaddexp(0, x); so alpha =
      1 / (1 + e^x).  (The pages compute the gates inside each chunk -- "Hybrid
      Linear Attention Architectures...", Hardware-Aware Chunkwise
      Parallelism, implementation checklist -- without printing the
      activation; this is the log-sigmoid reading.)
    * "scalar"   -- one alpha per token and head, [...], applied to every key
      channel: the scalar gate of Gated DeltaNet ("Hybrid Linear Attention
      Architectures...", Core Module Design, Stage 2).
    """
    g = _f64(gate)
    if kind == "alpha":
        return g
    if kind == "softplus":
        return np.exp(-np.logaddexp(0.0, g))
    if kind == "scalar":
        return np.repeat(g[..., None], Dk, axis=-1)
    raise ValueError(kind)


def kda_fwd(q, k, v, alpha, beta, initial_state=None, cu_seqlens=None,
            nthreads: int = 0, return_threads: bool = False):
    """Token-by-token KDA forward in fp64.

    q, k, alpha: [B, T, H, Dk]; v: [B, T, H, Dv]; beta: [B, T, H].
    initial_state: [N, H, Dk, Dv] or None (zeros).
    cu_seqlens: None (N = B sequences of length T) or int [N+1] with B == 1.
    Returns (o [B,T,H,Dv] float64, final_state [N,H,Dk,Dv] float64).
    """
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or alpha.shape != q.shape or v.shape[:3] != q.shape[:3] \
            or beta.shape != q.shape[:3]:
        raise ValueError("oracle: inconsistent input shapes")
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        if B != 1 or cu.ndim != 1 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
            raise ValueError("oracle: bad cu_seqlens")
        N = cu.shape[0] - 1
        cu_p = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    else:
        cu = None
        N = B
        cu_p = None
    s0 = None
    if initial_state is not None:
        s0 = _f64(initial_state)
        if s0.shape != (N, H, Dk, Dv):
            raise ValueError("oracle: initial_state shape")
    o = np.zeros((B, T, H, Dv), dtype=np.float64)
    sT = np.zeros((N, H, Dk, Dv), dtype=np.float64)
    used = ctypes.c_int(0)
    rc = _load().kda_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                _ptr(s0), _ptr(sT), cu_p, N, _ptr(o), B, T, H, Dk, Dv,
                                int(nthreads), ctypes.byref(used))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_fwd failed: {rc}")
    if return_threads:
        return o, sT, used.value
    return o, sT


def kda_step(q, k, v, alpha, beta, state, nthreads: int = 0, return_threads: bool = False):
    """One recurrent decode step in fp64.

    q, k, alpha: [N, H, Dk]; v: [N, H, Dv]; beta: [N, H]; state: [N, H, Dk, Dv].
    Returns (o [N,H,Dv], new_state); the input ``state`` is not modified.
    """
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    if st.shape != (N, H, Dk, Dv) or beta.shape != (N, H):
        raise ValueError("oracle: inconsistent step shapes")
    o = np.zeros((N, H, Dv), dtype=np.float64)
    used = ctypes.c_int(0)
    rc = _load().kda_oracle_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                 _ptr(st), _ptr(o), N, H, Dk, Dv, int(nthreads),
                                 ctypes.byref(used))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_step failed: {rc}")
    if return_threads:
        return o, st, used.value
    return o, st


def _cu_arg(cu_seqlens, B, T):
    if cu_seqlens is None:
        return None, B, None
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    if B != 1 or cu.ndim != 1 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("oracle: bad cu_seqlens")
    return cu, cu.shape[0] - 1, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def kda_bwd(q, k, v, alpha, beta, dout, initial_state=None, dfinal_state=None,
            cu_seqlens=None, nthreads: int = 0):
    """Gradients of L = sum(dout * o) + sum(dfinal_state * S_T) in fp64.

    Same inputs as ``kda_fwd`` plus dout [B,T,H,Dv] and dfinal_state
    [N,H,Dk,Dv] (None = zeros).  Returns a dict with dq, dk [B,T,H,Dk],
    dv [B,T,H,Dv], dalpha [B,T,H,Dk] (per channel), dbeta [B,T,H] and
    dinitial_state [N,H,Dk,Dv] (dL/dS_0; meaningful whether or not an
    initial state was given, zeros standing in for a missing one).
    """
    q, k, v, alpha, beta, dout = map(_f64, (q, k, v, alpha, beta, dout))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or alpha.shape != q.shape or v.shape[:3] != q.shape[:3] \
            or beta.shape != q.shape[:3] or dout.shape != v.shape:
        raise ValueError("oracle: inconsistent input shapes")
    cu, N, cu_p = _cu_arg(cu_seqlens, B, T)
    s0 = None if initial_state is None else _f64(initial_state)
    dsT = None if dfinal_state is None else _f64(dfinal_state)
    for x in (s0, dsT):
        if x is not None and x.shape != (N, H, Dk, Dv):
            raise ValueError("oracle: state shape")
    r = dict(dq=np.zeros((B, T, H, Dk)), dk=np.zeros((B, T, H, Dk)), dv=np.zeros((B, T, H, Dv)),
             dalpha=np.zeros((B, T, H, Dk)), dbeta=np.zeros((B, T, H)),
             dinitial_state=np.zeros((N, H, Dk, Dv)))
    used = ctypes.c_int(0)
    rc = _load().kda_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(s0),
                                cu_p, N, _ptr(dout), _ptr(dsT), _ptr(r["dq"]), _ptr(r["dk"]),
                                _ptr(r["dv"]), _ptr(r["dalpha"]), _ptr(r["dbeta"]),
                                _ptr(r["dinitial_state"]), B, T, H, Dk, Dv, int(nthreads),
                                ctypes.byref(used))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_bwd failed: {rc}")
    r["threads"] = used.value
    return r


def gate_grad(dalpha, gate, kind: str):
    """dL/d(gate) in the form ``kind`` from the per-channel dL/dalpha.

    * "alpha"    -- dalpha itself.
    * "softplus" -- alpha = 1 / (1 + e^x), so dalpha/dx = -alpha (1 - alpha),
      evaluated as -sigmoid(x) sigmoid(-x).
    * "scalar"   -- the one gate feeds every key channel: the channel
      gradients add up.
    """
    da = _f64(dalpha)
    if kind == "alpha":
        return da
    if kind == "softplus":
        x = _f64(gate)
        return -da * np.exp(-np.logaddexp(0.0, x)) * np.exp(-np.logaddexp(0.0, -x))
    if kind == "scalar":
        return da.sum(axis=-1)
    raise ValueError(kind)
