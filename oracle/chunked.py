"""Chunkwise KDA forward in numpy fp64 -- TEST INFRASTRUCTURE ONLY (part of the oracle).

Follows the chunked algorithm of "Linear Attention KDA Gating in a 3:1 Hybrid
Architecture: Principles and Implementation Guide", section 3 (3.1 inter-chunk
state transition, 3.2 intra-chunk output with causal masking), and the
"Hardware-Aware Chunkwise Parallelism" section of "Hybrid Linear Attention
Architectures...", with these readings of the garbled passages:

* Gamma_r is the inclusive product of alpha over the chunk's first r tokens,
  per key channel (a C x d_k array); gamma = Gamma_c is the whole-chunk decay.
  The state-update factor of token r is gamma / Gamma_r.
* W and U are per-token rows (C x d_k and C x d_v).  For the chunk update
  "S_next = Diag(gamma) S + (factor * K)^T (U - W S)" to equal the recurrence
  for every incoming S, they must be
      A = strictly-lower( Diag(beta) (Gamma*K) (K/Gamma)^T ),
      W = (I + A)^-1 Diag(beta) (Gamma*K),
      U = (I + A)^-1 Diag(beta) V,
  i.e. the unit-lower-triangular solve the printed pseudocode leaves out
  (the printed sums are not dimensionally consistent).
* Tril keeps the diagonal: token i sees tokens j <= i.
* A partial last chunk is simply shorter (no padding is needed in fp64).

The inverse (I + A)^-1 is applied with a library triangular solve; everything
else is written out step by step in the order the pages give.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def chunk_intermediates(q, k, v, alpha, beta, S):
    """All per-chunk quantities for one chunk of one head.

    q, k, alpha: [c, Dk]; v: [c, Dv]; beta: [c]; S: [Dk, Dv] (state entering
    the chunk).  Returns a dict with b (cumulative log-decay), Gamma, gamma,
    A, W, U, Uc (= U - W S), P (= Tril(Qhat Kbar^T)), O and S_next.
    """
    q, k, v, alpha, beta, S = (np.asarray(x, dtype=np.float64) for x in (q, k, v, alpha, beta, S))
    c = q.shape[0]
    b = np.cumsum(np.log(alpha), axis=0)          # log-domain accumulation
    Gamma = np.exp(b)                               # [c, Dk], decay from chunk start through r
    gamma = Gamma[-1]                               # whole-chunk decay, [Dk]
    Qh = Gamma * q                                  # Gamma (.) Q
    Kh = Gamma * k                                  # Gamma (.) K
    Kb = k * np.exp(-b)                             # K / Gamma
    Kt = k * np.exp(b[-1][None, :] - b)             # (gamma / Gamma) (.) K
    A = np.tril(beta[:, None] * (Kh @ Kb.T), -1)
    IA = np.eye(c) + A
    W = solve_triangular(IA, beta[:, None] * Kh, lower=True, unit_diagonal=True)
    U = solve_triangular(IA, beta[:, None] * v, lower=True, unit_diagonal=True)
    Uc = U - W @ S
    P = np.tril(Qh @ Kb.T)
    O = Qh @ S + P @ Uc
    S_next = gamma[:, None] * S + Kt.T @ Uc
    return dict(b=b, Gamma=Gamma, gamma=gamma, Qh=Qh, Kh=Kh, Kb=Kb, Kt=Kt, A=A,
                W=W, U=U, Uc=Uc, P=P, O=O, S_next=S_next)


def kda_fwd_chunked(q, k, v, alpha, beta, initial_state=None, cu_seqlens=None, chunk_size=64):
    """Chunkwise forward with the same interface as ``oracle.kda_fwd``."""
    q, k, v, alpha, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, alpha, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if cu_seqlens is None:
        seqs = [(bb, 0, T) for bb in range(B)]
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        assert B == 1
        seqs = [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    N = len(seqs)
    o = np.zeros((B, T, H, Dv))
    sT = np.zeros((N, H, Dk, Dv))
    for n, (bb, t0, t1) in enumerate(seqs):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if initial_state is None else np.array(initial_state[n, h], dtype=np.float64)
            for c0 in range(t0, t1, chunk_size):
                c1 = min(c0 + chunk_size, t1)
                r = chunk_intermediates(q[bb, c0:c1, h], k[bb, c0:c1, h], v[bb, c0:c1, h],
                                        alpha[bb, c0:c1, h], beta[bb, c0:c1, h], S)
                o[bb, c0:c1, h] = r["O"]
                S = r["S_next"]
            sT[n, h] = S
    return o, sT


def chunk_grads(q, k, v, alpha, beta, S, dO, dS_next):
    """Backward of one chunk's map (S, inputs) -> (O, S_next) of ``chunk_intermediates``.

    dO: [c, Dv] gradient of the chunk's outputs; dS_next: [Dk, Dv] gradient of
    the state leaving the chunk.  Returns a dict with dq, dk, dalpha ([c, Dk]),
    dv ([c, Dv]), dbeta ([c]), dS (gradient of the state entering the chunk)
    and dUc (= dL/d(U - W S)).

    Each step is the chain rule through one line of the forward, in reverse:
      O = Qh S + P Uc,  S_next = Diag(gamma) S + Kt^T Uc,  Uc = U - W S,
      P = Tril(Qh Kb^T),  W = T Y,  U = T Z  (T = (I + A)^-1, Y = Diag(beta) Kh,
      Z = Diag(beta) V),  A = StrictTril(Diag(beta) Kh Kb^T),
      Qh = Gamma Q, Kh = Gamma K, Kb = K / Gamma, Kt = (gamma / Gamma) K,
      Gamma = exp(b), b = cumsum(log alpha).
    """
    r = chunk_intermediates(q, k, v, alpha, beta, S)
    q, k, v, alpha, beta, S, dO, dS_next = (np.asarray(x, dtype=np.float64)
                                            for x in (q, k, v, alpha, beta, S, dO, dS_next))
    c = q.shape[0]
    Qh, Kh, Kb, Kt, W, Uc, P = r["Qh"], r["Kh"], r["Kb"], r["Kt"], r["W"], r["Uc"], r["P"]
    Gamma, gamma = r["Gamma"], r["gamma"]
    T = solve_triangular(np.eye(c) + r["A"], np.eye(c), lower=True, unit_diagonal=True)

    # the state pass (reverse): gradients of Uc and of the incoming state
    dUc = P.T @ dO + Kt @ dS_next
    dS = gamma[:, None] * dS_next + Qh.T @ dO - W.T @ dUc
    # O = Qh S + P Uc;  P = Tril(Qh Kb^T)
    M = np.tril(dO @ Uc.T)                       # dP, masked like P
    dQh = dO @ S.T + M @ Kb
    dKb = M.T @ Qh
    # S_next = Diag(gamma) S + Kt^T Uc;  Uc = U - W S
    dKt = Uc @ dS_next.T
    dgamma = np.sum(dS_next * S, axis=1)
    dW = -dUc @ S.T
    dU = dUc
    # W = T Y, U = T Z
    Y = beta[:, None] * Kh
    dT = dW @ Y.T + dU @ (beta[:, None] * v).T
    dY = T.T @ dW
    dZ = T.T @ dU
    dv = beta[:, None] * dZ
    dbeta = np.sum(dZ * v, axis=1) + np.sum(dY * Kh, axis=1)
    dKh = beta[:, None] * dY
    # T = (I + A)^-1:  dA = -T^T dT T^T, kept where A lives (strictly lower)
    dA = np.tril(-T.T @ dT @ T.T, -1)
    R = Kh @ Kb.T
    dbeta += np.sum(dA * R, axis=1)
    dR = beta[:, None] * dA
    dKh += dR @ Kb
    dKb += dR.T @ Kh
    # gates
    dq = Gamma * dQh
    dk = Gamma * dKh + dKb / Gamma + (gamma[None, :] / Gamma) * dKt
    db = Qh * dQh + Kh * dKh - Kb * dKb - Kt * dKt
    db[-1] += gamma * dgamma + np.sum(Kt * dKt, axis=0)
    dg = np.cumsum(db[::-1], axis=0)[::-1]       # b_r = sum_{s <= r} log alpha_s
    dalpha = dg / alpha
    return dict(dq=dq, dk=dk, dv=dv, dalpha=dalpha, dbeta=dbeta, dS=dS, dUc=dUc)


def kda_bwd_chunked(q, k, v, alpha, beta, dout, initial_state=None, dfinal_state=None,
                    cu_seqlens=None, chunk_size=64):
    """Chunkwise backward with the same interface and result as ``oracle.kda_bwd``:
    a forward pass over the chunks records the state entering each chunk, then
    the chunks are differentiated last to first, the state gradient flowing
    backwards between them."""
    q, k, v, alpha, beta, dout = (np.asarray(x, dtype=np.float64)
                                  for x in (q, k, v, alpha, beta, dout))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if cu_seqlens is None:
        seqs = [(bb, 0, T) for bb in range(B)]
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        assert B == 1
        seqs = [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    N = len(seqs)
    out = dict(dq=np.zeros((B, T, H, Dk)), dk=np.zeros((B, T, H, Dk)), dv=np.zeros((B, T, H, Dv)),
               dalpha=np.zeros((B, T, H, Dk)), dbeta=np.zeros((B, T, H)),
               dinitial_state=np.zeros((N, H, Dk, Dv)))
    for n, (bb, t0, t1) in enumerate(seqs):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if initial_state is None else np.array(initial_state[n, h], dtype=np.float64)
            bounds, states = [], []
            for c0 in range(t0, t1, chunk_size):
                c1 = min(c0 + chunk_size, t1)
                bounds.append((c0, c1))
                states.append(S)
                S = chunk_intermediates(q[bb, c0:c1, h], k[bb, c0:c1, h], v[bb, c0:c1, h],
                                        alpha[bb, c0:c1, h], beta[bb, c0:c1, h], S)["S_next"]
            dS = np.zeros((Dk, Dv)) if dfinal_state is None else np.array(dfinal_state[n, h], dtype=np.float64)
            for (c0, c1), S_in in zip(reversed(bounds), reversed(states)):
                g = chunk_grads(q[bb, c0:c1, h], k[bb, c0:c1, h], v[bb, c0:c1, h],
                                alpha[bb, c0:c1, h], beta[bb, c0:c1, h], S_in,
                                dout[bb, c0:c1, h], dS)
                for key in ("dq", "dk", "dv", "dalpha", "dbeta"):
                    out[key][bb, c0:c1, h] = g[key]
                dS = g["dS"]
            out["dinitial_state"][n, h] = dS
    return out
