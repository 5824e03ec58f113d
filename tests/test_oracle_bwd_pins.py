"""Pins of the oracle's backward (``oracle.kda_bwd``, ``oracle.gate_grad``,
``oracle.chunked.kda_bwd_chunked``).

The backward is the vector-Jacobian product of the recurrence of "Hybrid
Linear Attention Architectures...", Core Module Design, Stage 3, for
L = sum(dO * o) + sum(dS_T * S_T).  What fixes it independently of the
oracle's own chain-rule code:

* central finite differences of the (already pinned) forward oracle;
* closed forms of a degenerate case (alpha = 1, beta = 0: the state never
  changes, so o_t = S_0^T q_t and everything is a plain sum);
* linearity of a vector-Jacobian product in the upstream gradient;
* the state-split property: differentiating [0, T) equals differentiating
  [T1, T) and then [0, T1) with the state gradient handed across;
* the chunkwise form ("Linear Attention KDA Gating...", sections 3.1 and 3.2,
  differentiated chunk by chunk) against the token recurrence, any chunk size.
"""
import numpy as np
import pytest

import oracle
from oracle.chunked import kda_bwd_chunked

RNG = np.random.default_rng(20261204)
NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "dinitial_state")


def inputs(B, T, H, Dk, Dv, N=None, mu=-2.0, rng=RNG):
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    alpha = np.exp(-np.logaddexp(0.0, rng.standard_normal((B, T, H, Dk)) + mu))
    N = B if N is None else N
    S0 = rng.standard_normal((N, H, Dk, Dv))
    dO = rng.standard_normal((B, T, H, Dv))
    dST = rng.standard_normal((N, H, Dk, Dv))
    return q, k, v, alpha, beta, S0, dO, dST


def loss(args, dO, dST, cu=None):
    q, k, v, alpha, beta, S0 = args
    o, sT = oracle.kda_fwd(q, k, v, alpha, beta, initial_state=S0, cu_seqlens=cu)
    return float(np.sum(o * dO) + np.sum(sT * dST))


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# Every gradient against central differences (step 1e-6, error O(h^2) plus
# cancellation ~1e-10), with packed sequences including an empty one.
def test_bwd_matches_finite_differences():
    cu = [0, 4, 4, 9]
    q, k, v, alpha, beta, S0, dO, dST = inputs(1, 9, 2, 3, 2, N=3)
    args = [q, k, v, alpha, beta, S0]
    r = oracle.kda_bwd(q, k, v, alpha, beta, dO, S0, dST, cu_seqlens=cu)
    h = 1e-6
    for i, name in enumerate(NAMES):
        fd = np.zeros_like(args[i])
        for idx in np.ndindex(args[i].shape):
            ap = [x.copy() for x in args]
            am = [x.copy() for x in args]
            ap[i][idx] += h
            am[i][idx] -= h
            fd[idx] = (loss(ap, dO, dST, cu) - loss(am, dO, dST, cu)) / (2 * h)
        assert rel(r[name], fd) < 1e-7, name
    # the empty sequence passes its state gradient straight through
    assert np.array_equal(r["dinitial_state"][1], dST[1])


# alpha = 1, beta = 0: S_t = S_0 for all t ("Hybrid Linear Attention
# Architectures...", the DeltaNet form with a zero learning rate), so
#   dq_t = S_0 dO_t,  dk = dv = 0,  G_t = dS_T + sum_{s >= t} q_s dO_s^T,
#   dbeta_t = k_t^T G_t (v_t - S_0^T k_t),  dalpha_t = rowsum(G_t * S_0),
#   dS_0 = dS_T + sum_t q_t dO_t^T.
def test_bwd_closed_form_frozen_state():
    T, Dk, Dv = 11, 5, 4
    q, k, v, _, _, S0, dO, dST = inputs(1, T, 1, Dk, Dv)
    r = oracle.kda_bwd(q, k, v, np.ones((1, T, 1, Dk)), np.zeros((1, T, 1)), dO, S0, dST)
    S, Q, K, V, G0 = S0[0, 0], q[0, :, 0], k[0, :, 0], v[0, :, 0], dO[0, :, 0]
    assert np.max(np.abs(r["dq"][0, :, 0] - G0 @ S.T)) < 1e-13
    assert np.all(r["dk"] == 0) and np.all(r["dv"] == 0)
    for t in range(T):
        G = dST[0, 0] + Q[t:].T @ G0[t:]
        assert abs(r["dbeta"][0, t, 0] - K[t] @ G @ (V[t] - S.T @ K[t])) < 1e-12
        assert np.max(np.abs(r["dalpha"][0, t, 0] - np.sum(G * S, axis=1))) < 1e-12
    assert np.max(np.abs(r["dinitial_state"][0, 0] - (dST[0, 0] + Q.T @ G0))) < 1e-12


def test_bwd_is_linear_in_upstream_gradient():
    q, k, v, alpha, beta, S0, dO1, dS1 = inputs(2, 20, 2, 6, 4)
    dO2 = RNG.standard_normal(dO1.shape)
    dS2 = RNG.standard_normal(dS1.shape)
    a, b = 1.3, -0.6
    r1 = oracle.kda_bwd(q, k, v, alpha, beta, dO1, S0, dS1)
    r2 = oracle.kda_bwd(q, k, v, alpha, beta, dO2, S0, dS2)
    r3 = oracle.kda_bwd(q, k, v, alpha, beta, a * dO1 + b * dO2, S0, a * dS1 + b * dS2)
    for name in NAMES:
        assert rel(r3[name], a * r1[name] + b * r2[name]) < 1e-12, name


# Chain rule across a split of the sequence ("Linear Attention KDA Gating...",
# section 3.1: the state is the only thing carried between chunks).
def test_bwd_state_split():
    T, T1 = 70, 29
    q, k, v, alpha, beta, S0, dO, dST = inputs(1, T, 2, 6, 5)
    full = oracle.kda_bwd(q, k, v, alpha, beta, dO, S0, dST)
    sl1, sl2 = slice(0, T1), slice(T1, T)
    _, S1 = oracle.kda_fwd(q[:, sl1], k[:, sl1], v[:, sl1], alpha[:, sl1], beta[:, sl1],
                           initial_state=S0)
    second = oracle.kda_bwd(q[:, sl2], k[:, sl2], v[:, sl2], alpha[:, sl2], beta[:, sl2],
                            dO[:, sl2], S1, dST)
    first = oracle.kda_bwd(q[:, sl1], k[:, sl1], v[:, sl1], alpha[:, sl1], beta[:, sl1],
                           dO[:, sl1], S0, second["dinitial_state"])
    for name in NAMES[:5]:
        joined = np.concatenate([first[name], second[name]], axis=1)
        assert rel(joined, full[name]) < 1e-12, name
    assert rel(first["dinitial_state"], full["dinitial_state"]) < 1e-12


@pytest.mark.parametrize("C", [1, 2, 7, 16, 64])
def test_bwd_chunked_equals_recurrence(C):
    cu = [0, 37, 37, 100, 101]
    q, k, v, alpha, beta, S0, dO, dST = inputs(1, 101, 2, 8, 6, N=4)
    ref = oracle.kda_bwd(q, k, v, alpha, beta, dO, S0, dST, cu_seqlens=cu)
    got = kda_bwd_chunked(q, k, v, alpha, beta, dO, S0, dST, cu_seqlens=cu, chunk_size=C)
    for name in NAMES:
        assert rel(got[name], ref[name]) < 1e-13, (C, name)


def test_bwd_without_state_arguments_is_zero_state():
    q, k, v, alpha, beta, _, dO, _ = inputs(2, 10, 1, 4, 4)
    z = np.zeros((2, 1, 4, 4))
    r1 = oracle.kda_bwd(q, k, v, alpha, beta, dO)
    r2 = oracle.kda_bwd(q, k, v, alpha, beta, dO, z, z)
    for name in NAMES:
        assert np.array_equal(r1[name], r2[name]), name


def test_bwd_threads_do_not_change_results():
    q, k, v, alpha, beta, S0, dO, dST = inputs(2, 40, 3, 8, 8)
    r1 = oracle.kda_bwd(q, k, v, alpha, beta, dO, S0, dST, nthreads=1)
    r8 = oracle.kda_bwd(q, k, v, alpha, beta, dO, S0, dST, nthreads=8)
    for name in NAMES:
        assert np.array_equal(r1[name], r8[name]), name


# gate_grad: the chain rule from dalpha to each gate form, against central
# differences of the forward oracle through alpha_from_gate.
@pytest.mark.parametrize("kind", ["softplus", "scalar"])
def test_gate_grad_matches_finite_differences(kind):
    T, Dk, Dv = 6, 3, 2
    q, k, v, _, beta, S0, dO, dST = inputs(1, T, 1, Dk, Dv)
    shape = (1, T, 1, Dk) if kind == "softplus" else (1, T, 1)
    gate = RNG.standard_normal(shape) - 1.0 if kind == "softplus" else RNG.uniform(0.5, 1.0, shape)
    alpha = oracle.alpha_from_gate(gate, kind, Dk)
    r = oracle.kda_bwd(q, k, v, alpha, beta, dO, S0, dST)
    got = oracle.gate_grad(r["dalpha"], gate, kind)
    assert got.shape == gate.shape
    h = 1e-6
    fd = np.zeros_like(gate)
    for idx in np.ndindex(gate.shape):
        gp, gm = gate.copy(), gate.copy()
        gp[idx] += h
        gm[idx] -= h
        lp = loss([q, k, v, oracle.alpha_from_gate(gp, kind, Dk), beta, S0], dO, dST)
        lm = loss([q, k, v, oracle.alpha_from_gate(gm, kind, Dk), beta, S0], dO, dST)
        fd[idx] = (lp - lm) / (2 * h)
    assert rel(got, fd) < 1e-7
