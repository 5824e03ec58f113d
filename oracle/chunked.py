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
