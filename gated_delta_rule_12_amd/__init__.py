"""Python binding of the KDA HIP library (``libkda.so``, gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/kda.h``.  PyTorch provides
device memory (outputs and workspace, when the caller does not pass them)
and the current HIP stream.  There is no fallback: when ``libkda.so`` is
missing the first call raises.

Functions carry the C names:

* ``kda_chunk_fwd``                 chunkwise forward (prefill / training forward)
* ``kda_chunk_fwd_gated``           the same with the gate in any ``kda_gate`` form
* ``kda_chunk_fwd_static``          the same on the library's static workspace (no allocation)
* ``kda_chunk_fwd_workspace_bytes`` workspace size of a chunkwise forward
* ``kda_chunk_bwd``                 chunkwise backward (training): all input gradients
* ``kda_chunk_bwd_workspace_bytes`` workspace size of a chunkwise backward
* ``kda_recurrent_step``            one decode step, state updated in place
* ``kda_recurrent_step_gated``      the same with the gate in any ``kda_gate`` form
* ``kda_status_string``             name of a status code

The Python ``kda_chunk_fwd`` / ``kda_recurrent_step`` take ``gate=`` ("alpha",
"softplus" or "scalar") and call the ``*_gated`` entry points for the other
two forms.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_SUCCESS = 0
KDA_ERROR_INVALID_VALUE = 1
KDA_ERROR_NOT_SUPPORTED = 2
KDA_ERROR_WORKSPACE_TOO_SMALL = 3
KDA_ERROR_LAUNCH = 4

KDA_DTYPE_F32 = 0
KDA_DTYPE_BF16 = 1

KDA_GATE_ALPHA = 0
KDA_GATE_SOFTPLUS_BF16 = 1
KDA_GATE_SCALAR = 2
_GATES = {"alpha": KDA_GATE_ALPHA, "softplus": KDA_GATE_SOFTPLUS_BF16, "scalar": KDA_GATE_SCALAR}

EXPORTED = ("kda_status_string", "kda_chunk_fwd_workspace_bytes", "kda_chunk_fwd",
            "kda_chunk_fwd_gated", "kda_chunk_fwd_static", "kda_chunk_bwd_workspace_bytes",
            "kda_chunk_bwd", "kda_recurrent_step", "kda_recurrent_step_gated")

# size of the static workspace of kda_chunk_fwd_static (KDA_STATIC_WORKSPACE_BYTES)
KDA_STATIC_WORKSPACE_BYTES = 64 << 20

_lib = None


class KDAError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {kda_status_string(status)} ({status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded ``libkda.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"KDA HIP library not built: {LIB_PATH} is missing "
                               "(run __graft_entry__.build() or gated_delta_rule_12_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        L.kda_status_string.restype = ctypes.c_char_p
        L.kda_status_string.argtypes = [i32]
        L.kda_chunk_fwd_workspace_bytes.restype = sz
        L.kda_chunk_fwd_workspace_bytes.argtypes = [i32, i64, i32, i32, i32, i32, i32, i32, i32]
        L.kda_chunk_fwd.restype = i32
        L.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                    i32, i64, i32, i32, i32, i32, i32, i32, vp, sz, vp]
        L.kda_chunk_fwd_gated.restype = i32
        L.kda_chunk_fwd_gated.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, vp, i32, vp,
                                          i32, i64, i32, i32, i32, i32, i32, i32, vp, sz, vp]
        L.kda_chunk_fwd_static.restype = i32
        L.kda_chunk_fwd_static.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, vp, i32, vp,
                                           i32, i64, i32, i32, i32, i32, i32, i32, vp]
        L.kda_chunk_bwd_workspace_bytes.restype = sz
        L.kda_chunk_bwd_workspace_bytes.argtypes = [i32, i64, i32, i32, i32, i32, i32, i32, i32]
        L.kda_chunk_bwd.restype = i32
        L.kda_chunk_bwd.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, i32, vp, vp,
                                    vp, vp, vp, vp, vp, vp,
                                    i32, i64, i32, i32, i32, i32, i32, vp, sz, vp]
        L.kda_recurrent_step.restype = i32
        L.kda_recurrent_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                         i32, i32, vp]
        L.kda_recurrent_step_gated.restype = i32
        L.kda_recurrent_step_gated.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, i32, i32, i32,
                                               i32, i32, i32, vp]
        _lib = L
    return _lib


def kda_status_string(status: int) -> str:
    return lib().kda_status_string(int(status)).decode()


def _dt(t: torch.dtype) -> int:
    if t == torch.float32:
        return KDA_DTYPE_F32
    if t == torch.bfloat16:
        return KDA_DTYPE_BF16
    raise ValueError(f"unsupported dtype {t}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("KDA tensors must be contiguous")
    return t.data_ptr() or None


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _gate_spec(gate: str, lead: tuple, Dk: int):
    """(dtype, shape) of the forget gate in the form ``gate``."""
    if gate == "alpha":
        return torch.float32, tuple(lead) + (Dk,)
    if gate == "softplus":
        return torch.bfloat16, tuple(lead) + (Dk,)
    if gate == "scalar":
        return torch.float32, tuple(lead)
    raise ValueError(f"unknown gate form {gate!r}")


def _check(dev, what: str, t: Optional[torch.Tensor], dtype, shape):
    """``t`` (when given) is a GPU tensor on ``dev`` of this dtype and shape.
    The kernels read raw memory, so a wrong device, dtype or shape must never
    reach them."""
    if t is None:
        return
    _need(isinstance(t, torch.Tensor), f"{what}: expected a tensor")
    _need(t.is_cuda and t.device == dev, f"{what}: must be on {dev} (got {t.device})")
    _need(t.dtype == dtype, f"{what}: dtype {t.dtype}, expected {dtype}")
    _need(tuple(t.shape) == tuple(shape), f"{what}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_inputs(q, k, v, alpha, beta, gate, initial_state, cu_seqlens, N):
    """Shapes, dtypes and devices shared by the forward and backward calls."""
    _need(isinstance(q, torch.Tensor) and q.dim() == 4, "q: expected [B, T, H, Dk]")
    _need(q.is_cuda, "q: must be a GPU tensor")
    _need(q.dtype in (torch.float32, torch.bfloat16), f"q: unsupported dtype {q.dtype}")
    dev = q.device
    B, T, H, Dk = q.shape
    _check(dev, "k", k, q.dtype, q.shape)
    _need(isinstance(v, torch.Tensor) and v.dim() == 4, "v: expected [B, T, H, Dv]")
    _check(dev, "v", v, q.dtype, (B, T, H, v.shape[-1]))
    gdt, gshape = _gate_spec(gate, (B, T, H), Dk)
    _check(dev, f"gate ({gate})", alpha, gdt, gshape)
    _check(dev, "beta", beta, torch.float32, (B, T, H))
    _check(dev, "initial_state", initial_state, torch.float32, (N, H, Dk, v.shape[-1]))
    if cu_seqlens is not None:
        _check(dev, "cu_seqlens", cu_seqlens, torch.int32, (N + 1,))
        _need(B == 1, "cu_seqlens: packed sequences need B == 1")
    return dev


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _scratch(nbytes: int, dev, stream) -> torch.Tensor:
    """A workspace from torch's caching allocator.  When the call runs on a
    stream other than the current one, the block is recorded on that stream
    so that the allocator does not hand it out again while the call's
    kernels may still use it."""
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if stream is not None:
        s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream), device=dev)
        if s != torch.cuda.current_stream(dev):
            ws.record_stream(s)
    return ws


def _fwd_outputs(q, k, v, alpha, beta, initial_state, final_state, cu_seqlens, o, out_dtype, gate):
    """Check the forward's inputs and return (o, final_state or None, N),
    allocating the outputs that were not given."""
    N = q.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
    dev = _check_inputs(q, k, v, alpha, beta, gate, initial_state, cu_seqlens, N)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if out_dtype is None:
        out_dtype = q.dtype if o is None else o.dtype
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=out_dtype, device=dev)
    _check(dev, "o", o, out_dtype, (B, T, H, Dv))
    if final_state is True:
        final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev)
    elif final_state is False:
        final_state = None
    _check(dev, "final_state", final_state, torch.float32, (N, H, Dk, Dv))
    return o, final_state, N


def kda_chunk_fwd_workspace_bytes(B: int, T: int, H: int, Dk: int, Dv: int, varlen: bool,
                                  num_seqs: int, chunk_size: int, act_dtype) -> int:
    dt = act_dtype if isinstance(act_dtype, int) else _dt(act_dtype)
    return int(lib().kda_chunk_fwd_workspace_bytes(B, T, H, Dk, Dv, int(bool(varlen)),
                                                   num_seqs, chunk_size, dt))


def kda_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                  beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                  final_state=None, cu_seqlens: Optional[torch.Tensor] = None,
                  o: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                  workspace: Optional[torch.Tensor] = None, chunk_size: int = 64,
                  stream=None, gate: str = "alpha") -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise KDA forward on the GPU.

    q, k [B,T,H,Dk]; v [B,T,H,Dv]; beta [B,T,H]; initial_state
    [N,H,Dk,Dv] fp32 or None; cu_seqlens int32 [N+1] (B == 1) or None.
    ``alpha`` is the forget gate in the form ``gate``: "alpha" (fp32
    [B,T,H,Dk]), "softplus" (bf16 pre-activation x [B,T,H,Dk], log alpha =
    -softplus(x)) or "scalar" (fp32 [B,T,H], one alpha per token and head).
    ``final_state``: None (not computed), True (allocate) or an fp32 tensor
    [N,H,Dk,Dv] (may be ``initial_state`` itself, updated in place).
    Returns (o, final_state or None).
    """
    o, final_state, N = _fwd_outputs(q, k, v, alpha, beta, initial_state, final_state,
                                     cu_seqlens, o, out_dtype, gate)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    act = _dt(q.dtype)
    dev = q.device
    sid = _stream(stream)
    need = kda_chunk_fwd_workspace_bytes(B, T, H, Dk, Dv, cu_seqlens is not None, N,
                                         chunk_size, act)
    if workspace is None and need > 0:
        workspace = _scratch(need, dev, stream)
    elif workspace is not None:
        _check(dev, "workspace", workspace, torch.uint8, (workspace.numel(),))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    g = _GATES[gate]
    if g == KDA_GATE_ALPHA:
        st = lib().kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                 _ptr(initial_state), _ptr(final_state), _ptr(cu_seqlens), N,
                                 _ptr(o), B, T, H, Dk, Dv, chunk_size, act, _dt(o.dtype),
                                 _ptr(workspace), ws_bytes, sid)
        where = "kda_chunk_fwd"
    else:
        st = lib().kda_chunk_fwd_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), g, _ptr(beta),
                                       _ptr(initial_state), _ptr(final_state), _ptr(cu_seqlens), N,
                                       _ptr(o), B, T, H, Dk, Dv, chunk_size, act, _dt(o.dtype),
                                       _ptr(workspace), ws_bytes, sid)
        where = "kda_chunk_fwd_gated"
    if st != KDA_SUCCESS:
        raise KDAError(st, where)
    return o, final_state


def kda_chunk_fwd_static(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                         beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                         final_state=None, cu_seqlens: Optional[torch.Tensor] = None,
                         o: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                         chunk_size: int = 64, stream=None,
                         gate: str = "alpha") -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``kda_chunk_fwd`` on the library's static workspace: the C call
    allocates nothing (pass ``o`` and ``final_state`` to allocate nothing at
    all).  Problems needing more than KDA_STATIC_WORKSPACE_BYTES of workspace
    raise KDA_ERROR_WORKSPACE_TOO_SMALL.  Calls that may overlap on one GPU
    share that workspace and must be ordered by the caller."""
    o, final_state, N = _fwd_outputs(q, k, v, alpha, beta, initial_state, final_state,
                                     cu_seqlens, o, out_dtype, gate)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    st = lib().kda_chunk_fwd_static(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _GATES[gate], _ptr(beta),
                                    _ptr(initial_state), _ptr(final_state), _ptr(cu_seqlens), N,
                                    _ptr(o), B, T, H, Dk, Dv, chunk_size, _dt(q.dtype), _dt(o.dtype),
                                    _stream(stream))
    if st != KDA_SUCCESS:
        raise KDAError(st, "kda_chunk_fwd_static")
    return o, final_state


def kda_chunk_bwd_workspace_bytes(B: int, T: int, H: int, Dk: int, Dv: int, varlen: bool,
                                  num_seqs: int, chunk_size: int, act_dtype) -> int:
    dt = act_dtype if isinstance(act_dtype, int) else _dt(act_dtype)
    return int(lib().kda_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, int(bool(varlen)),
                                                   num_seqs, chunk_size, dt))


def kda_chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                  beta: torch.Tensor, dout: torch.Tensor,
                  initial_state: Optional[torch.Tensor] = None,
                  dfinal_state: Optional[torch.Tensor] = None,
                  cu_seqlens: Optional[torch.Tensor] = None, need_dinitial_state: bool = True,
                  workspace: Optional[torch.Tensor] = None, chunk_size: int = 64, stream=None,
                  gate: str = "alpha", out: Optional[dict] = None) -> dict:
    """Chunkwise KDA backward on the GPU: gradients of
    L = sum(dout * o) + sum(dfinal_state * S_T) for the forward with the same
    inputs (see kda_chunk_fwd; ``alpha`` is the gate in the form ``gate``).

    dout [B,T,H,Dv] in the dtype of q; dfinal_state [N,H,Dk,Dv] fp32 or None.
    Returns a dict with dq, dk (like q), dv (like v), dgate (fp32, the shape
    of ``alpha``), dbeta (fp32 [B,T,H]) and dinitial_state (fp32 [N,H,Dk,Dv],
    or None when ``need_dinitial_state`` is False).  ``out`` may hold
    preallocated tensors under those names.
    """
    N = q.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
    dev = _check_inputs(q, k, v, alpha, beta, gate, initial_state, cu_seqlens, N)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    act = _dt(q.dtype)
    _check(dev, "dout", dout, q.dtype, v.shape)
    _check(dev, "dfinal_state", dfinal_state, torch.float32, (N, H, Dk, Dv))
    r = dict(out) if out else {}
    r.setdefault("dq", torch.empty_like(q))
    r.setdefault("dk", torch.empty_like(k))
    r.setdefault("dv", torch.empty_like(v))
    r.setdefault("dgate", torch.empty(alpha.shape, dtype=torch.float32, device=dev))
    r.setdefault("dbeta", torch.empty(beta.shape, dtype=torch.float32, device=dev))
    if need_dinitial_state:
        r.setdefault("dinitial_state", torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev))
    else:
        r["dinitial_state"] = None
    gdt, gshape = _gate_spec(gate, (B, T, H), Dk)
    for key, dt, shp in (("dq", q.dtype, q.shape), ("dk", q.dtype, q.shape), ("dv", q.dtype, v.shape),
                         ("dgate", torch.float32, gshape), ("dbeta", torch.float32, (B, T, H))):
        _check(dev, key, r[key], dt, shp)
    _check(dev, "dinitial_state", r["dinitial_state"], torch.float32, (N, H, Dk, Dv))
    need = kda_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, cu_seqlens is not None, N, chunk_size, act)
    if workspace is None and need > 0:
        workspace = _scratch(need, dev, stream)
    elif workspace is not None:
        _check(dev, "workspace", workspace, torch.uint8, (workspace.numel(),))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().kda_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _GATES[gate], _ptr(beta),
                             _ptr(initial_state), _ptr(cu_seqlens), N, _ptr(dout),
                             _ptr(dfinal_state), _ptr(r["dq"]), _ptr(r["dk"]), _ptr(r["dv"]),
                             _ptr(r["dgate"]), _ptr(r["dbeta"]), _ptr(r["dinitial_state"]),
                             B, T, H, Dk, Dv, chunk_size, act, _ptr(workspace), ws_bytes,
                             _stream(stream))
    if st != KDA_SUCCESS:
        raise KDAError(st, "kda_chunk_bwd")
    return r


def kda_recurrent_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                       beta: torch.Tensor, state: torch.Tensor, o: Optional[torch.Tensor] = None,
                       out_dtype: Optional[torch.dtype] = None, stream=None,
                       gate: str = "alpha") -> torch.Tensor:
    """One KDA decode step on the GPU; ``state`` [N,H,Dk,Dv] fp32 is updated in place.

    q, k [N,H,Dk]; v [N,H,Dv]; beta [N,H]; ``alpha`` in the form ``gate``
    (as for kda_chunk_fwd: [N,H,Dk], or [N,H] for "scalar").  Returns o [N,H,Dv].
    """
    _need(isinstance(q, torch.Tensor) and q.dim() == 3 and q.is_cuda, "q: expected a GPU tensor [N, H, Dk]")
    _need(q.dtype in (torch.float32, torch.bfloat16), f"q: unsupported dtype {q.dtype}")
    dev = q.device
    N, H, Dk = q.shape
    _need(isinstance(v, torch.Tensor) and v.dim() == 3, "v: expected [N, H, Dv]")
    Dv = v.shape[-1]
    _check(dev, "k", k, q.dtype, q.shape)
    _check(dev, "v", v, q.dtype, (N, H, Dv))
    gdt, gshape = _gate_spec(gate, (N, H), Dk)
    _check(dev, f"gate ({gate})", alpha, gdt, gshape)
    _check(dev, "beta", beta, torch.float32, (N, H))
    _check(dev, "state", state, torch.float32, (N, H, Dk, Dv))
    if out_dtype is None:
        out_dtype = q.dtype if o is None else o.dtype
    if o is None:
        o = torch.empty((N, H, Dv), dtype=out_dtype, device=dev)
    _check(dev, "o", o, out_dtype, (N, H, Dv))
    g = _GATES[gate]
    if g == KDA_GATE_ALPHA:
        st = lib().kda_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                      _ptr(state), _ptr(o), N, H, Dk, Dv, _dt(q.dtype),
                                      _dt(o.dtype), _stream(stream))
        where = "kda_recurrent_step"
    else:
        st = lib().kda_recurrent_step_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), g, _ptr(beta),
                                            _ptr(state), _ptr(o), N, H, Dk, Dv, _dt(q.dtype),
                                            _dt(o.dtype), _stream(stream))
        where = "kda_recurrent_step_gated"
    if st != KDA_SUCCESS:
        raise KDAError(st, where)
    return o
