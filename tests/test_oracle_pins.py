"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test names the passage it follows.  None of them re-types the oracle's
own expanded arithmetic: they use a hand-worked example, exact rational
arithmetic on the literal matrix form, closed forms of special cases,
invariants, O(N^2) brute force and equivalences between formulations.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.chunked import chunk_intermediates, kda_fwd_chunked

RNG = np.random.default_rng(20261203)


def rand_inputs(B, T, H, Dk, Dv, rng=RNG, unit=True, mu=-2.0):
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    alpha = np.exp(-np.log1p(np.exp(rng.standard_normal((B, T, H, Dk)) + mu)))
    return q, k, v, alpha, beta


# ---------------------------------------------------------------------------
# Hand-worked example (tests/golden/kda_hand_example.txt): the KDA update rule
# of "Hybrid Linear Attention Architectures...", Core Module Design, Stage 3.
# ---------------------------------------------------------------------------
def test_hand_worked_example(golden):
    g = golden("kda_hand_example.txt")
    sq = tuple(int(x) for x in g["shape_qk"])
    sv = tuple(int(x) for x in g["shape_v"])
    ss = tuple(int(x) for x in g["shape_state"])
    o, sT = oracle.kda_fwd(g["q"].reshape(sq), g["k"].reshape(sq), g["v"].reshape(sv),
                           g["alpha"].reshape(sq), g["beta"].reshape(sq[:3]),
                           initial_state=g["initial_state"].reshape(ss))
    assert np.array_equal(o.ravel(), g["expected_o"])
    assert np.array_equal(sT.ravel(), g["expected_final_state"])


# ---------------------------------------------------------------------------
# P1: the literal matrix form (I - b k k^T) Diag(a) S + b k v^T, o = S^T q, in
# exact rational arithmetic on small random rationals.  Same source as above.
# ---------------------------------------------------------------------------
def _frac_matmul(A, B):
    return [[sum((A[i][t] * B[t][j] for t in range(len(B))), Fraction(0))
             for j in range(len(B[0]))] for i in range(len(A))]


def _literal_exact(q, k, v, a, b, S0):
    Dk, Dv = len(S0), len(S0[0])
    S = [row[:] for row in S0]
    outs = []
    for t in range(len(q)):
        E = [[(Fraction(1) if i == j else Fraction(0)) - b[t] * k[t][i] * k[t][j]
              for j in range(Dk)] for i in range(Dk)]
        D = [[a[t][i] if i == j else Fraction(0) for j in range(Dk)] for i in range(Dk)]
        S = _frac_matmul(_frac_matmul(E, D), S)
        S = [[S[i][j] + b[t] * k[t][i] * v[t][j] for j in range(Dv)] for i in range(Dk)]
        outs.append([sum((S[i][j] * q[t][i] for i in range(Dk)), Fraction(0)) for j in range(Dv)])
    return outs, S


def test_literal_matrix_form_exact_rationals():
    rng = np.random.default_rng(1)
    T, Dk, Dv = 6, 3, 4

    def r(*shape, lo=-8, hi=9, den=8):
        return [[Fraction(int(x), den) for x in row] for row in rng.integers(lo, hi, size=shape)]

    q, k, v = r(T, Dk), r(T, Dk), r(T, Dv)
    a = [[Fraction(int(x), 16) for x in row] for row in rng.integers(1, 17, size=(T, Dk))]
    b = [Fraction(int(x), 8) for x in rng.integers(0, 9, size=T)]
    S0 = r(Dk, Dv)
    outs, S = _literal_exact(q, k, v, a, b, S0)

    f = lambda M: np.array([[float(x) for x in row] for row in M])
    o, sT = oracle.kda_fwd(f(q)[None, :, None], f(k)[None, :, None], f(v)[None, :, None],
                           f(a)[None, :, None], np.array([float(x) for x in b])[None, :, None],
                           initial_state=f(S0)[None, None])
    ref_o, ref_s = f(outs), f(S)
    assert np.max(np.abs(o[0, :, 0] - ref_o)) <= 1e-13 * max(1.0, np.max(np.abs(ref_o)))
    assert np.max(np.abs(sT[0, 0] - ref_s)) <= 1e-13 * max(1.0, np.max(np.abs(ref_s)))


# ---------------------------------------------------------------------------
# P2: with alpha = 1, S0 = 0 and a vanishing write strength beta = eps, the
# state is eps * sum_s k_s v_s^T + O(eps^2): plain causal linear attention
# ("Hybrid Linear Attention Architectures...", Stage 1; "Linear Attention
# KDA Gating...", section 2, item 1).  Checked against O(N^2) brute force.
# ---------------------------------------------------------------------------
def test_linear_attention_limit_bruteforce():
    q, k, v, _, _ = rand_inputs(1, 40, 2, 8, 5)
    alpha = np.ones_like(q)
    eps = 1e-9
    beta = np.full(q.shape[:3], eps)
    o, _ = oracle.kda_fwd(q, k, v, alpha, beta)
    ref = np.zeros_like(o)
    for h in range(2):
        for t in range(40):
            for s in range(t + 1):                      # causal, diagonal included
                ref[0, t, h] += np.dot(q[0, t, h], k[0, s, h]) * v[0, s, h]
    err = np.max(np.abs(o / eps - ref)) / np.max(np.abs(ref))
    assert err < 1e-6


# P3: literal beta = 0 (no write at all): o_t = S0^T q_t and the state only decays.
def test_beta_zero_reads_initial_state():
    q, k, v, _, _ = rand_inputs(1, 9, 3, 6, 7)
    S0 = RNG.standard_normal((1, 3, 6, 7))
    alpha = np.ones_like(q)
    o, sT = oracle.kda_fwd(q, k, v, alpha, np.zeros(q.shape[:3]), initial_state=S0)
    ref = np.einsum("thc,hcj->thj", q[0], S0[0])
    assert np.max(np.abs(o[0] - ref)) < 1e-14
    assert np.array_equal(sT, S0)


# ---------------------------------------------------------------------------
# P4 (DeltaNet, alpha = 1): "subtract the old value first, then write the new
# one" ("Hybrid Linear Attention Architectures...", Stage 1; "Designing and
# Deploying Hybrid MLA...", section 2, Step 2).
# ---------------------------------------------------------------------------
def test_deltanet_readback_exact_overwrite():
    # beta = 1 and |k| = 1: the memory returns exactly v_t for key k_t, so
    # with q_t = k_t the output is v_t.
    q, k, v, _, _ = rand_inputs(1, 30, 2, 16, 9)
    S0 = RNG.standard_normal((1, 2, 16, 9))
    o, _ = oracle.kda_fwd(k, k, v, np.ones_like(k), np.ones(k.shape[:3]), initial_state=S0)
    assert np.max(np.abs(o - v)) < 1e-13


def test_deltanet_householder_preserves_norm():
    # beta = 2, v = 0, |k| = 1: I - 2 k k^T is a reflection, so ||S||_F is kept.
    q, k, _, _, _ = rand_inputs(1, 50, 1, 12, 7)
    S0 = RNG.standard_normal((1, 1, 12, 7))
    _, sT = oracle.kda_fwd(q, k, np.zeros((1, 50, 1, 7)), np.ones_like(k),
                           np.full((1, 50, 1), 2.0), initial_state=S0)
    assert abs(np.linalg.norm(sT) - np.linalg.norm(S0)) < 1e-12 * np.linalg.norm(S0)


def test_basis_keys_closed_form():
    # k_t = e_j: every row decays by its own alpha, then row j becomes
    # (1 - beta) * (decayed row j) + beta * v_t^T.  (KDA with per-channel decay.)
    T, Dk, Dv = 25, 5, 3
    js = RNG.integers(0, Dk, size=T)
    k = np.zeros((1, T, 1, Dk))
    k[0, np.arange(T), 0, js] = 1.0
    q = RNG.standard_normal((1, T, 1, Dk))
    v = RNG.standard_normal((1, T, 1, Dv))
    alpha = RNG.uniform(0.3, 1.0, size=(1, T, 1, Dk))
    beta = RNG.uniform(0.0, 1.0, size=(1, T, 1))
    S = RNG.standard_normal((Dk, Dv))
    o, sT = oracle.kda_fwd(q, k, v, alpha, beta, initial_state=S[None, None])
    for t in range(T):
        S = alpha[0, t, 0][:, None] * S
        j = js[t]
        S[j] = (1.0 - beta[0, t, 0]) * S[j] + beta[0, t, 0] * v[0, t, 0]
        assert np.max(np.abs(o[0, t, 0] - q[0, t, 0] @ S)) < 1e-13
    assert np.max(np.abs(sT[0, 0] - S)) < 1e-13


# ---------------------------------------------------------------------------
# P5: operator order -- decay first, then the key-direction overwrite
# ("Linear Attention KDA Gating...", section 2, item 5).  With non-uniform
# alpha, beta = 1 and unit k the read-back o_t = v_t (q_t = k_t) holds only
# for decay-first; the opposite order would scale the written value.
# ---------------------------------------------------------------------------
def test_operator_order_decay_first():
    q, k, v, alpha, _ = rand_inputs(1, 40, 2, 16, 8, mu=-1.0)
    assert np.ptp(alpha) > 0.3
    S0 = RNG.standard_normal((1, 2, 16, 8))
    o, _ = oracle.kda_fwd(k, k, v, alpha, np.ones(k.shape[:3]), initial_state=S0)
    assert np.max(np.abs(o - v)) < 1e-13


# P6: Dk != Dv -- shapes and the read-back through o.
def test_rectangular_state():
    q, k, v, alpha, beta = rand_inputs(2, 11, 3, 8, 5)
    o, sT = oracle.kda_fwd(q, k, v, alpha, beta)
    assert o.shape == (2, 11, 3, 5) and sT.shape == (2, 3, 8, 5)
    o2, _ = oracle.kda_fwd(k, k, v, alpha, np.ones(k.shape[:3]))
    assert np.max(np.abs(o2 - v)) < 1e-13


# ---------------------------------------------------------------------------
# P7: the chunkwise form ("Linear Attention KDA Gating...", sections 3.1 and
# 3.2) equals the recurrence for every chunk size, including a ragged tail.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("C", [1, 2, 3, 7, 16, 64])
def test_chunked_equals_recurrence(C):
    q, k, v, alpha, beta = rand_inputs(2, 37, 2, 8, 6)
    S0 = 0.3 * RNG.standard_normal((2, 2, 8, 6))
    o_r, s_r = oracle.kda_fwd(q, k, v, alpha, beta, initial_state=S0)
    o_c, s_c = kda_fwd_chunked(q, k, v, alpha, beta, initial_state=S0, chunk_size=C)
    assert np.max(np.abs(o_c - o_r)) < 1e-12
    assert np.max(np.abs(s_c - s_r)) < 1e-12


def test_chunk_intermediates_structure():
    # A is strictly lower triangular; (I + A) W = Diag(beta) (Gamma*K); the
    # chunk state update equals the recurrence run over the chunk.
    q, k, v, alpha, beta = rand_inputs(1, 16, 1, 6, 4)
    S = RNG.standard_normal((6, 4))
    r = chunk_intermediates(q[0, :, 0], k[0, :, 0], v[0, :, 0], alpha[0, :, 0], beta[0, :, 0], S)
    assert np.all(np.triu(r["A"]) == 0)
    lhs = (np.eye(16) + r["A"]) @ r["W"]
    assert np.max(np.abs(lhs - beta[0, :, 0, None] * r["Kh"])) < 1e-13
    o, sT = oracle.kda_fwd(q, k, v, alpha, beta, initial_state=S[None, None])
    assert np.max(np.abs(r["S_next"] - sT[0, 0])) < 1e-13
    assert np.max(np.abs(r["O"] - o[0, :, 0])) < 1e-13


# ---------------------------------------------------------------------------
# P8: the state in/out is the resume mechanism -- splitting a sequence and
# carrying S across the split changes nothing; packed (cu_seqlens) batches
# equal separate runs ("pass the inter-chunk state matrix S from one chunk to
# the next", "Hybrid Linear Attention Architectures...", implementation
# checklist).
# ---------------------------------------------------------------------------
def test_state_split_is_exact():
    q, k, v, alpha, beta = rand_inputs(1, 50, 2, 8, 8)
    S0 = RNG.standard_normal((1, 2, 8, 8))
    o, sT = oracle.kda_fwd(q, k, v, alpha, beta, initial_state=S0)
    o1, s1 = oracle.kda_fwd(q[:, :17], k[:, :17], v[:, :17], alpha[:, :17], beta[:, :17], initial_state=S0)
    o2, s2 = oracle.kda_fwd(q[:, 17:], k[:, 17:], v[:, 17:], alpha[:, 17:], beta[:, 17:], initial_state=s1)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), o)
    assert np.array_equal(s2, sT)


def test_varlen_equals_separate_sequences():
    lens = [5, 0, 13, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v, alpha, beta = rand_inputs(1, T, 3, 8, 4)
    S0 = RNG.standard_normal((len(lens), 3, 8, 4))
    o, sT = oracle.kda_fwd(q, k, v, alpha, beta, initial_state=S0, cu_seqlens=cu)
    for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        on, sn = oracle.kda_fwd(q[:, a:b], k[:, a:b], v[:, a:b], alpha[:, a:b], beta[:, a:b],
                                initial_state=S0[n:n + 1])
        assert np.array_equal(o[:, a:b], on)
        assert np.array_equal(sT[n], sn[0])
    assert np.array_equal(sT[1], S0[1])                  # empty sequence: final = initial


def test_batch_rows_and_heads_are_independent():
    q, k, v, alpha, beta = rand_inputs(3, 12, 4, 8, 8)
    o, sT = oracle.kda_fwd(q, k, v, alpha, beta)
    for b in range(3):
        for h in range(4):
            sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
            ob, sb = oracle.kda_fwd(q[sl], k[sl], v[sl], alpha[sl], beta[sl])
            assert np.array_equal(ob[0, :, 0], o[b, :, h])
            assert np.array_equal(sb[0, 0], sT[b, h])


# P9: T decode steps equal one forward over T tokens (recurrent kernels for
# decode: "Linear Attention + Sparse Attention...", section 6).
def test_decode_steps_equal_forward():
    N, T, H, D = 3, 7, 2, 8
    q, k, v, alpha, beta = rand_inputs(N, T, H, D, D)
    S0 = RNG.standard_normal((N, H, D, D))
    o, sT = oracle.kda_fwd(q, k, v, alpha, beta, initial_state=S0)
    st = S0.copy()
    for t in range(T):
        ot, st = oracle.kda_step(q[:, t], k[:, t], v[:, t], alpha[:, t], beta[:, t], st)
        assert np.array_equal(ot, o[:, t])
    assert np.array_equal(st, sT)


# P10: o and S_T are jointly linear in (V, S0) -- the update is affine in S
# with a write term linear in v.
def test_linearity_in_values_and_state():
    q, k, v1, alpha, beta = rand_inputs(1, 20, 2, 8, 6)
    v2 = RNG.standard_normal(v1.shape)
    S1, S2 = RNG.standard_normal((2, 1, 2, 8, 6))
    a, b = 0.7, -1.9
    o1, s1 = oracle.kda_fwd(q, k, v1, alpha, beta, initial_state=S1)
    o2, s2 = oracle.kda_fwd(q, k, v2, alpha, beta, initial_state=S2)
    o3, s3 = oracle.kda_fwd(q, k, a * v1 + b * v2, alpha, beta, initial_state=a * S1 + b * S2)
    assert np.max(np.abs(o3 - (a * o1 + b * o2))) < 1e-12
    assert np.max(np.abs(s3 - (a * s1 + b * s2))) < 1e-12


# P11: a channel-uniform gate alpha_t = a_t 1 gives the gated DeltaNet form
# S_t = a_t (I - b k k^T) S + b k v^T ("Hybrid Linear Attention
# Architectures...", Stage 2; for a scalar gate both operator orders agree).
def test_scalar_gate_is_gated_deltanet():
    T, Dk, Dv = 15, 6, 5
    q, k, v, _, beta = rand_inputs(1, T, 1, Dk, Dv)
    a = RNG.uniform(0.5, 1.0, size=T)
    alpha = np.broadcast_to(a[None, :, None, None], (1, T, 1, Dk)).copy()
    S = RNG.standard_normal((Dk, Dv))
    o, sT = oracle.kda_fwd(q, k, v, alpha, beta, initial_state=S[None, None])
    for t in range(T):
        kt, bt = k[0, t, 0], beta[0, t, 0]
        S = a[t] * (np.eye(Dk) - bt * np.outer(kt, kt)) @ S + bt * np.outer(kt, v[0, t, 0])
        assert np.max(np.abs(o[0, t, 0] - S.T @ q[0, t, 0])) < 1e-13


# Gate forms of the library's gate= argument (oracle.alpha_from_gate).
# Pre-activation form: log alpha = -softplus(x) is alpha = 1 / (1 + e^x)
# (the closed form, not the oracle's logaddexp), with alpha(0) = 1/2, alpha
# falling in x, alpha -> 1 for x -> -inf (where KDA becomes DeltaNet, P4) and
# alpha ~ e^-x for large x.
def test_gate_softplus_closed_form():
    x = np.array([-60.0, -20.0, -3.5, -1.0, -0.25, 0.0, 0.5, 2.0, 7.0, 30.0])
    a = oracle.alpha_from_gate(x, "softplus", 1)
    assert np.max(np.abs(a / (1.0 / (1.0 + np.exp(x))) - 1.0)) < 1e-14
    assert a[5] == 0.5 and a[0] == 1.0
    assert np.all(np.diff(a) < 0)
    assert abs(a[-1] / np.exp(-30.0) - 1.0) < 1e-12


def test_gate_softplus_limit_is_deltanet():
    q, k, v, _, beta = rand_inputs(1, 20, 2, 6, 5)
    S0 = RNG.standard_normal((1, 2, 6, 5))
    x = np.full((1, 20, 2, 6), -60.0)
    o1, s1 = oracle.kda_fwd(q, k, v, oracle.alpha_from_gate(x, "softplus", 6), beta, initial_state=S0)
    o2, s2 = oracle.kda_fwd(q, k, v, np.ones((1, 20, 2, 6)), beta, initial_state=S0)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


# Scalar form: one alpha per (token, head) on every key channel; through the
# recurrence it is the gated DeltaNet update of P11.
def test_gate_scalar_is_gated_deltanet():
    T, Dk, Dv = 12, 5, 4
    q, k, v, _, beta = rand_inputs(1, T, 1, Dk, Dv)
    a = RNG.uniform(0.4, 1.0, size=(1, T, 1))
    alpha = oracle.alpha_from_gate(a, "scalar", Dk)
    assert alpha.shape == (1, T, 1, Dk) and np.all(alpha == a[..., None])
    S = RNG.standard_normal((Dk, Dv))
    o, _ = oracle.kda_fwd(q, k, v, alpha, beta, initial_state=S[None, None])
    for t in range(T):
        kt, bt = k[0, t, 0], beta[0, t, 0]
        S = a[0, t, 0] * (np.eye(Dk) - bt * np.outer(kt, kt)) @ S + bt * np.outer(kt, v[0, t, 0])
        assert np.max(np.abs(o[0, t, 0] - S.T @ q[0, t, 0])) < 1e-13


def test_threads_do_not_change_results():
    q, k, v, alpha, beta = rand_inputs(2, 33, 5, 8, 8)
    o1, s1, n1 = oracle.kda_fwd(q, k, v, alpha, beta, nthreads=1, return_threads=True)
    o8, s8, n8 = oracle.kda_fwd(q, k, v, alpha, beta, nthreads=8, return_threads=True)
    assert n1 == 1 and n8 == 8
    assert np.array_equal(o1, o8) and np.array_equal(s1, s8)


def test_oracle_rejects_bad_shapes():
    q, k, v, alpha, beta = rand_inputs(1, 4, 1, 4, 4)
    with pytest.raises(ValueError):
        oracle.kda_fwd(q, k[:, :3], v, alpha, beta)
    with pytest.raises(ValueError):
        oracle.kda_fwd(q, k, v, alpha, beta, cu_seqlens=[0, 2, 3])   # does not end at T
