"""Pins of the fp64 oracle to facts other than itself (CPU only).

Each test checks the oracle against something the pages or plain mathematics
fix: worked examples printed on the pages (tests/golden), exact rational
brute force with explicit transition matrices, closed forms of special cases,
invariants of the update, and library routines for reductions to textbook
operations.  A plausible slip in the oracle (a dropped term, a wrong sign, the
fade applied after the read, a transposed operand, the output read before the
write) fails at least one of them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import golden
from gated_delta_rule_08_amd import workloads


def _one_head(arrs):
    """[T, d] single-head arrays -> [T, 1, d] packed layout."""
    return [None if a is None else np.asarray(a, dtype=np.float64)[:, None] for a in arrs]


def _run1(q, k, v, g, beta, s0=None, mode=oracle.MODE_DELTA):
    q, k, v, g = _one_head((q, k, v, g))
    beta = np.asarray(beta, dtype=np.float64).reshape(-1, 1)
    if s0 is not None:
        s0 = np.asarray(s0, dtype=np.float64)[None, None]
    o, s = oracle.run(q, k, v, g, beta, s0=s0, mode=mode, nthreads=1)
    return o[:, 0], s[0, 0]


# ---------------------------------------------------------------- worked examples

def test_whiteboard_additive_read():
    """Additive memory read equals the page's hand-checked [2, 2.8, 0.6, 2.2]."""
    f = golden.load("whiteboard_additive_read.txt")
    k = np.stack([f["k1"], f["k2"]])
    v = np.stack([f["v1"], f["v2"]])
    q = np.stack([f["q"], f["q"]])
    g = np.zeros((2, 4))
    o, S = _run1(q, k, v, g, np.ones(2), mode=oracle.MODE_ADDITIVE)
    np.testing.assert_allclose(o[1], f["read"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[1] - f["v1"], f["crosstalk"], rtol=0, atol=1e-14)
    # before Rex is written the cat read is clean
    np.testing.assert_allclose(o[0], f["v1"], rtol=0, atol=1e-14)


def test_delta_overwrite_worked_example():
    """beta = 1 overwrite turns row 0 into exactly [1, 0, 2, 2]; row 2 untouched."""
    f = golden.load("delta_overwrite.txt")
    S0 = np.zeros((4, 4))
    S0[0] = f["v_old"]
    S0[2] = [5.0, -3.0, 0.25, 7.0]   # another fact under key e2
    S0[1] = [0.5, 0.5, -1.0, 2.0]
    q = np.eye(4)[[0]]
    o, S = _run1(q, f["k"][None], f["v_new"][None], np.zeros((1, 4)), f["beta"], s0=S0)
    np.testing.assert_allclose(S[0], f["row0_after"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(S[0] - S0[0], f["u"], rtol=0, atol=1e-14)
    np.testing.assert_array_equal(S[1:], S0[1:])
    np.testing.assert_allclose(o[0], f["row0_after"], rtol=0, atol=1e-14)


def test_chunk_two_token_solve_worked_example():
    """Two tokens, beta = 1: the corrections are u1 = v1 and u2 = [-1.2, 2.4, 1, 1.4]."""
    f = golden.load("chunk_two_token_solve.txt")
    k = np.stack([f["k1"], f["k2"]])
    v = np.stack([f["v1"], f["v2"]])
    _, S = _run1(np.zeros((2, 4)), k, v, np.zeros((2, 4)), np.ones(2))
    expect = np.outer(f["k1"], f["u1"]) + np.outer(f["k2"], f["u2"])
    np.testing.assert_allclose(S, expect, rtol=0, atol=1e-14)
    # the last key now retrieves its value exactly
    np.testing.assert_allclose(f["k2"] @ S, f["v2"], rtol=0, atol=1e-14)


def test_survival_product_worked_example():
    """Gates 0.9, 0.5, 0.9 after a write leave 0.405 of the value (beta = 0 afterwards)."""
    f = golden.load("survival_product.txt")
    d = 4
    e0 = np.eye(d)[0]
    v = np.array([2.0, 1.0, 0.0, 1.0])
    T = 6
    k = np.tile(e0, (T, 1))
    q = np.tile(e0, (T, 1))
    vv = np.tile(v, (T, 1))
    beta = np.array([0, 0, 1, 0, 0, 0], dtype=np.float64)   # only step 3 writes
    g = np.zeros((T, d))
    g[3:] = np.log(f["gates"])[:, None]
    o, _ = _run1(q, k, vv, g, beta)
    np.testing.assert_allclose(o[5], f["strength"][0] * v, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(o[2], v, rtol=0, atol=1e-15)


# ---------------------------------------------------------------- (a) brute force

def _frac_matrix(rows):
    return [[Fraction(x) for x in r] for r in rows]


def _brute_force(alpha, beta, k, v, q, S0, order="fade_first", convention="rows_are_keys",
                 unfaded_read=False):
    """Exact rational recurrence with the transition matrix built explicitly.

    fade_first:  S_t = (I - b k k^T) Diag(a) S_{t-1} + b k v^T     (default)
    erase_first: S_t = Diag(a) (I - b k k^T) S_{t-1} + b k v^T
    unfaded_read: the read uses S_{t-1} before the fade (a listing variant).
    """
    T = len(beta)
    dk, dv = len(k[0]), len(v[0])
    S = [row[:] for row in S0]
    outs = []
    for t in range(T):
        a, b, kt, vt, qt = alpha[t], beta[t], k[t], v[t], q[t]
        E = [[(1 if i == j else 0) - b * kt[i] * kt[j] for j in range(dk)] for i in range(dk)]
        D = [[a[i] if i == j else 0 for j in range(dk)] for i in range(dk)]
        if unfaded_read:
            w = [sum(kt[r] * S[r][c] for r in range(dk)) for c in range(dv)]
            u = [b * (vt[c] - w[c]) for c in range(dv)]
            S = [[a[r] * S[r][c] + kt[r] * u[c] for c in range(dv)] for r in range(dk)]
        else:
            if order == "fade_first":
                M = [[sum(E[i][m] * D[m][j] for m in range(dk)) for j in range(dk)] for i in range(dk)]
            else:
                M = [[sum(D[i][m] * E[m][j] for m in range(dk)) for j in range(dk)] for i in range(dk)]
            S = [[sum(M[r][m] * S[m][c] for m in range(dk)) + b * kt[r] * vt[c] for c in range(dv)]
                 for r in range(dk)]
        if convention == "rows_are_keys":
            outs.append([sum(qt[r] * S[r][c] for r in range(dk)) for c in range(dv)])
    return outs, S


def _rational_problem(seed, T, dk, dv, scalar_gate=False):
    rng = np.random.default_rng(seed)
    def rq(lo, hi, den):
        return Fraction(int(rng.integers(lo, hi + 1)), den)
    alpha = []
    for _ in range(T):
        if scalar_gate:
            a = rq(1, 8, 8)
            alpha.append([a] * dk)
        else:
            alpha.append([rq(1, 8, 8) for _ in range(dk)])
    beta = [rq(0, 4, 4) for _ in range(T)]
    k = [[rq(-4, 4, 4) for _ in range(dk)] for _ in range(T)]
    v = [[rq(-6, 6, 3) for _ in range(dv)] for _ in range(T)]
    q = [[rq(-4, 4, 4) for _ in range(dk)] for _ in range(T)]
    S0 = [[rq(-5, 5, 5) for _ in range(dv)] for _ in range(dk)]
    return alpha, beta, k, v, q, S0


def _to_f(x):
    return np.array(x, dtype=np.float64)


def _oracle_on_rational(alpha, beta, k, v, q, S0):
    g = np.log(_to_f(alpha))
    return _run1(_to_f(q), _to_f(k), _to_f(v), g, _to_f(beta), s0=_to_f(S0))


@pytest.mark.parametrize("seed,T,dk,dv", [(1, 8, 4, 4), (2, 7, 3, 4), (3, 5, 4, 2), (4, 8, 2, 3)])
def test_brute_force_explicit_transition_matrices(seed, T, dk, dv):
    """Oracle == exact rational product of explicit (I - b k k^T) Diag(a) matrices."""
    alpha, beta, k, v, q, S0 = _rational_problem(seed, T, dk, dv)
    outs, S = _brute_force(alpha, beta, k, v, q, S0)
    o, Sf = _oracle_on_rational(alpha, beta, k, v, q, S0)
    scale = max(1.0, np.abs(_to_f(outs)).max())
    assert np.abs(o - _to_f(outs)).max() <= 1e-12 * scale
    assert np.abs(Sf - _to_f(S)).max() <= 1e-12 * max(1.0, np.abs(_to_f(S)).max())


def test_brute_force_unrolled_product():
    """S_T = (prod M) S_0 + sum_i (prod_{j>i} M_j) b_i k_i v_i^T, exactly."""
    T, dk, dv = 6, 3, 3
    alpha, beta, k, v, q, S0 = _rational_problem(11, T, dk, dv)

    def mat_mul(A, B):
        return [[sum(A[i][m] * B[m][j] for m in range(len(B))) for j in range(len(B[0]))]
                for i in range(len(A))]

    Ms = []
    for t in range(T):
        E = [[(1 if i == j else 0) - beta[t] * k[t][i] * k[t][j] for j in range(dk)] for i in range(dk)]
        D = [[alpha[t][i] if i == j else 0 for j in range(dk)] for i in range(dk)]
        Ms.append(mat_mul(E, D))
    ident = [[Fraction(1 if i == j else 0) for j in range(dk)] for i in range(dk)]

    def prod(lo, hi):  # M_{hi-1} ... M_lo
        P = ident
        for t in range(lo, hi):
            P = mat_mul(Ms[t], P)
        return P

    S = mat_mul(prod(0, T), S0)
    for i in range(T):
        W = [[beta[i] * k[i][r] * v[i][c] for c in range(dv)] for r in range(dk)]
        PW = mat_mul(prod(i + 1, T), W)
        S = [[S[r][c] + PW[r][c] for c in range(dv)] for r in range(dk)]
    _, Sf = _oracle_on_rational(alpha, beta, k, v, q, S0)
    assert np.abs(Sf - _to_f(S)).max() <= 1e-12 * max(1.0, np.abs(_to_f(S)).max())


def test_transposed_convention_gives_transposed_state():
    """The dv x dk column form S'(I - b k k^T)... is the transpose of the oracle's state."""
    T, dk, dv = 5, 3, 4
    alpha, beta, k, v, q, S0 = _rational_problem(21, T, dk, dv)
    Sp = [[S0[r][c] for r in range(dk)] for c in range(dv)]   # dv x dk
    for t in range(T):
        a, b, kt, vt = alpha[t], beta[t], k[t], v[t]
        # S' <- S' Diag(a) (I - b k k^T) + b v k^T
        SD = [[Sp[c][r] * a[r] for r in range(dk)] for c in range(dv)]
        E = [[(1 if i == j else 0) - b * kt[i] * kt[j] for j in range(dk)] for i in range(dk)]
        Sp = [[sum(SD[c][m] * E[m][r] for m in range(dk)) + b * vt[c] * kt[r] for r in range(dk)]
              for c in range(dv)]
    _, Sf = _oracle_on_rational(alpha, beta, k, v, q, S0)
    np.testing.assert_allclose(Sf.T, _to_f(Sp), rtol=1e-12, atol=1e-12)


def test_decay_order_reading():
    """Per-channel gates: fade-then-erase (used) differs from erase-then-fade;
    a scalar gate makes the two orders coincide."""
    T, dk, dv = 6, 4, 3
    alpha, beta, k, v, q, S0 = _rational_problem(31, T, dk, dv)
    _, S_fade_first = _brute_force(alpha, beta, k, v, q, S0, order="fade_first")
    _, S_erase_first = _brute_force(alpha, beta, k, v, q, S0, order="erase_first")
    _, Sf = _oracle_on_rational(alpha, beta, k, v, q, S0)
    assert np.abs(Sf - _to_f(S_fade_first)).max() < 1e-12
    assert np.abs(Sf - _to_f(S_erase_first)).max() > 1e-3
    alpha, beta, k, v, q, S0 = _rational_problem(32, T, dk, dv, scalar_gate=True)
    _, S1 = _brute_force(alpha, beta, k, v, q, S0, order="fade_first")
    _, S2 = _brute_force(alpha, beta, k, v, q, S0, order="erase_first")
    assert S1 == S2


def test_read_uses_faded_state():
    """The read is taken from the faded state; reading the unfaded state differs."""
    T, dk, dv = 6, 3, 3
    alpha, beta, k, v, q, S0 = _rational_problem(41, T, dk, dv, scalar_gate=True)
    _, S_unfaded = _brute_force(alpha, beta, k, v, q, S0, unfaded_read=True)
    _, Sf = _oracle_on_rational(alpha, beta, k, v, q, S0)
    assert np.abs(Sf - _to_f(S_unfaded)).max() > 1e-3


# ---------------------------------------------------------------- (b) beta = 0

def test_beta_zero_closed_form():
    """beta = 0: S_T = Diag(exp(sum_t g_t)) S_0 and o_t = (Diag(e^{G_t}) S_0)^T q_t."""
    rng = np.random.default_rng(5)
    T, dk, dv = 37, 8, 5
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    g = -rng.uniform(0, 0.3, (T, dk))
    S0 = rng.standard_normal((dk, dv))
    o, S = _run1(q, k, v, g, np.zeros(T), s0=S0)
    G = np.cumsum(g, axis=0)
    np.testing.assert_allclose(S, np.exp(G[-1])[:, None] * S0, rtol=1e-12, atol=1e-14)
    o_ref = np.stack([(np.exp(G[t])[:, None] * S0).T @ q[t] for t in range(T)])
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-13)


def test_idle_values_coast_untouched():
    """alpha = 1, beta = 0: the state is unchanged and every read is S_0^T q."""
    rng = np.random.default_rng(6)
    T, dk, dv = 9, 4, 6
    q = rng.standard_normal((T, dk))
    S0 = rng.standard_normal((dk, dv))
    o, S = _run1(q, rng.standard_normal((T, dk)), rng.standard_normal((T, dv)),
                 np.zeros((T, dk)), np.zeros(T), s0=S0)
    np.testing.assert_array_equal(S, S0)
    np.testing.assert_allclose(o, q @ S0, rtol=1e-13, atol=1e-14)


def test_wipe_with_strong_gate():
    """beta = 0 and a very small alpha wipe the memory."""
    rng = np.random.default_rng(7)
    S0 = rng.standard_normal((4, 4))
    o, S = _run1(rng.standard_normal((3, 4)), rng.standard_normal((3, 4)),
                 rng.standard_normal((3, 4)), np.full((3, 4), -30.0), np.zeros(3), s0=S0)
    assert np.abs(S).max() < 1e-30


# ---------------------------------------------------------------- (c) orthonormal keys

def test_orthonormal_keys_exact_retrieval():
    """alpha = 1, beta = 1, orthonormal keys: every written key reads back its value."""
    rng = np.random.default_rng(8)
    dk, dv, m = 16, 12, 11
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm.T[:m]
    vals = rng.standard_normal((m, dv))
    S0 = rng.standard_normal((dk, dv))
    _, S = _run1(np.zeros((m, dk)), keys, vals, np.zeros((m, dk)), np.ones(m), s0=S0)
    np.testing.assert_allclose(keys @ S, vals, rtol=0, atol=1e-12)
    # the directions never written keep the initial content
    rest = Qm.T[m:]
    np.testing.assert_allclose(rest @ S, rest @ S0, rtol=0, atol=1e-12)


def test_overwrite_same_key_returns_latest():
    rng = np.random.default_rng(9)
    dk, dv = 8, 5
    k = rng.standard_normal(dk)
    k /= np.linalg.norm(k)
    vals = rng.standard_normal((4, dv))
    _, S = _run1(np.zeros((4, dk)), np.tile(k, (4, 1)), vals, np.zeros((4, dk)), np.ones(4))
    np.testing.assert_allclose(k @ S, vals[-1], rtol=0, atol=1e-13)


def test_full_basis_overwrite_forgets_initial_state():
    """Writing a whole orthonormal basis with beta = 1 leaves S = sum k_i v_i^T."""
    rng = np.random.default_rng(10)
    d = 6
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = Qm.T
    vals = rng.standard_normal((d, d))
    _, S = _run1(np.zeros((d, d)), keys, vals, np.zeros((d, d)), np.ones(d),
                 s0=rng.standard_normal((d, d)))
    np.testing.assert_allclose(S, keys.T @ vals, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- (d) delta term disabled

def test_additive_mode_is_causal_linear_attention():
    """ADDITIVE, alpha = 1: O = tril(Q K^T) V, the causal prefix-sum read."""
    rng = np.random.default_rng(12)
    T, dk, dv = 40, 7, 9
    q, k, v = rng.standard_normal((T, dk)), rng.standard_normal((T, dk)), rng.standard_normal((T, dv))
    o, S = _run1(q, k, v, np.zeros((T, dk)), rng.uniform(0, 1, T), mode=oracle.MODE_ADDITIVE)
    np.testing.assert_allclose(o, np.tril(q @ k.T) @ v, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S, k.T @ v, rtol=1e-11, atol=1e-12)
    # prefix sums, step by step (the causal parallel view)
    Sp = np.cumsum(k[:, :, None] * v[:, None, :], axis=0)
    np.testing.assert_allclose(o, np.einsum("td,tde->te", q, Sp), rtol=1e-11, atol=1e-12)


def test_additive_mode_with_gate_closed_form():
    """ADDITIVE with per-channel gates: o_t = sum_{i<=t} ((q_t * e^{G_t-G_i}) . k_i) v_i
    plus the faded initial-state read."""
    rng = np.random.default_rng(13)
    T, dk, dv = 25, 6, 4
    q, k, v = rng.standard_normal((T, dk)), rng.standard_normal((T, dk)), rng.standard_normal((T, dv))
    g = -rng.uniform(0, 0.5, (T, dk))
    S0 = rng.standard_normal((dk, dv))
    o, S = _run1(q, k, v, g, np.zeros(T), s0=S0, mode=oracle.MODE_ADDITIVE)
    G = np.cumsum(g, axis=0)
    o_ref = np.zeros((T, dv))
    for t in range(T):
        o_ref[t] = (np.exp(G[t])[:, None] * S0).T @ q[t]
        for i in range(t + 1):
            o_ref[t] += np.dot(q[t] * np.exp(G[t] - G[i]), k[i]) * v[i]
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- invariants

def test_per_step_write_invariants():
    """Unit keys: k^T S_t = (1-b) k^T S̄_t + b v and |k^T S_t - v| = (1-b)|k^T S̄_t - v|;
    directions orthogonal to k are untouched by the erase."""
    rng = np.random.default_rng(14)
    T, dk, dv = 12, 8, 6
    prob = workloads.random_problem(rng, T, 1, dk, dv)
    q, k, v, g, beta = (prob[n][:, 0].astype(np.float64) for n in ("q", "k", "v", "g", "beta"))
    k = k / np.linalg.norm(k, axis=1, keepdims=True)
    S0 = rng.standard_normal((dk, dv))
    S_prev = S0
    for t in range(T):
        _, S_t = _run1(q[: t + 1], k[: t + 1], v[: t + 1], g[: t + 1], beta[: t + 1], s0=S0)
        Sbar = np.exp(g[t])[:, None] * S_prev
        lhs = k[t] @ S_t
        np.testing.assert_allclose(lhs, (1 - beta[t]) * (k[t] @ Sbar) + beta[t] * v[t],
                                   rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(np.linalg.norm(lhs - v[t]),
                                   (1 - beta[t]) * np.linalg.norm(k[t] @ Sbar - v[t]),
                                   rtol=1e-10, atol=1e-12)
        P = np.eye(dk) - np.outer(k[t], k[t])   # projector onto k's complement
        np.testing.assert_allclose(P @ S_t, P @ Sbar, rtol=1e-12, atol=1e-12)
        S_prev = S_t


def test_causality():
    """Perturbing any input after position t leaves o[<=t] bit-identical."""
    rng = np.random.default_rng(15)
    prob = workloads.random_problem(rng, 30, 2, 8, 8)
    o, _ = oracle.run(prob["q"], prob["k"], prob["v"], prob["g"], prob["beta"])
    t = 17
    p2 = {n: a.copy() for n, a in prob.items()}
    for n in ("q", "k", "v", "g"):
        p2[n][t + 1:] += rng.standard_normal(p2[n][t + 1:].shape).astype(np.float32) * 0.3
    p2["g"] = np.minimum(p2["g"], 0)
    p2["beta"][t + 1:] = 0.77
    o2, _ = oracle.run(p2["q"], p2["k"], p2["v"], p2["g"], p2["beta"])
    np.testing.assert_array_equal(o[: t + 1], o2[: t + 1])
    assert np.abs(o[t + 1:] - o2[t + 1:]).max() > 1e-3


def test_packed_sequences_are_independent_and_resumable():
    """Packed varlen == separate runs; run(a||b) == run(b) started from run(a)'s state."""
    rng = np.random.default_rng(16)
    lens = [5, 0, 13, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, d = int(cu[-1]), 3, 6
    prob = workloads.random_problem(rng, T, H, d, d)
    s0 = rng.standard_normal((len(lens), H, d, d))
    o, s = oracle.run(prob["q"], prob["k"], prob["v"], prob["g"], prob["beta"], cu, s0=s0)
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        on, sn = oracle.run(prob["q"][sl], prob["k"][sl], prob["v"][sl], prob["g"][sl],
                            prob["beta"][sl], s0=s0[n:n + 1])
        np.testing.assert_array_equal(o[sl], on)
        np.testing.assert_array_equal(s[n], sn[0])
    np.testing.assert_array_equal(s[1], s0[1])   # zero-length sequence keeps its state
    # split / resume
    sl = slice(cu[2], cu[3])
    a, b = slice(cu[2], cu[2] + 6), slice(cu[2] + 6, cu[3])
    _, sa = oracle.run(*(prob[n][a] for n in ("q", "k", "v", "g", "beta")), s0=s0[2:3])
    ob, sb = oracle.run(*(prob[n][b] for n in ("q", "k", "v", "g", "beta")), s0=sa)
    np.testing.assert_array_equal(ob, o[b])
    np.testing.assert_array_equal(sb[0], s[2])


def test_decode_equals_one_token_prefill():
    rng = np.random.default_rng(17)
    prob = workloads.random_problem(rng, 4, 2, 8, 8)
    s = rng.standard_normal((4, 2, 8, 8))
    o, sn = oracle.decode(prob["q"], prob["k"], prob["v"], prob["g"], prob["beta"], s)
    for b in range(4):
        ob, sb = oracle.run(*(prob[n][b:b + 1] for n in ("q", "k", "v", "g", "beta")), s0=s[b:b + 1])
        np.testing.assert_array_equal(o[b], ob[0])
        np.testing.assert_array_equal(sn[b], sb[0])


def test_threads_do_not_change_results():
    rng = np.random.default_rng(18)
    prob = workloads.random_problem(rng, 50, 5, 16, 16)
    cu = np.array([0, 20, 50], dtype=np.int32)
    o1, s1 = oracle.run(prob["q"], prob["k"], prob["v"], prob["g"], prob["beta"], cu, nthreads=1)
    o8, s8 = oracle.run(prob["q"], prob["k"], prob["v"], prob["g"], prob["beta"], cu, nthreads=8)
    np.testing.assert_array_equal(o1, o8)
    np.testing.assert_array_equal(s1, s8)


# ------------------------------------------------- input preparation (from raw projections)

def test_prepare_silu_normalize_closed_form():
    """normalize(silu(x)): silu(1) = 1/(1+e^-1), silu(-1) = -e^-1/(1+e^-1); the row is
    divided by its Euclidean norm; a zero row stays zero (the normaliser's floor)."""
    s1 = 1.0 / (1.0 + math.exp(-1.0))
    sm1 = -1.0 / (1.0 + math.exp(1.0))
    n = math.hypot(s1, sm1)
    q, k, g, beta = oracle.prepare_inputs(np.array([[1.0, -1.0], [0.0, 0.0]]),
                                          np.array([[3.0, 4.0], [-2.0, 0.5]]), gate="none")
    assert q[0, 0] == pytest.approx(s1 / n, rel=1e-15) and q[0, 1] == pytest.approx(sm1 / n, rel=1e-15)
    assert np.all(q[1] == 0.0)
    assert np.allclose(np.linalg.norm(k, axis=-1), 1.0, rtol=0, atol=1e-15)
    assert np.all(g == 0.0) and np.all(beta == 1.0)


def test_prepare_gates_closed_forms():
    """sigmoid(ln 3) = 3/4 exactly; log-sigmoid(0) = -ln 2; log-sigmoid(-50) = -50 - log1p(e^-50)
    and log-sigmoid(50) = -log1p(e^-50) without overflow or rounding to 0; the floor."""
    logits = np.array([0.0, math.log(3.0), -50.0, 50.0])
    _, _, g, beta = oracle.prepare_inputs(np.ones((4, 2)), np.ones((4, 2)),
                                          gate_logits=np.repeat(logits[:, None], 2, axis=1),
                                          beta_logits=logits)
    assert beta[1] == pytest.approx(0.75, rel=1e-15) and beta[0] == 0.5
    assert g[0, 0] == pytest.approx(-math.log(2.0), rel=1e-15)
    assert g[1, 0] == pytest.approx(math.log(0.75), rel=1e-15)
    assert g[2, 0] == pytest.approx(-50.0 - math.log1p(math.exp(-50.0)), rel=1e-15)
    assert g[3, 0] == pytest.approx(-math.exp(-50.0), rel=1e-12) and g[3, 0] < 0.0
    _, _, gf, _ = oracle.prepare_inputs(np.ones((4, 2)), np.ones((4, 2)),
                                        gate_logits=np.repeat(logits[:, None], 2, axis=1),
                                        beta_logits=logits, gate_min=-5.0)
    assert np.all(gf >= -5.0) and gf[2, 0] == -5.0 and gf[0, 0] == g[0, 0]


def test_prepare_scalar_gate_broadcasts():
    """A scalar gate logit per (token, head) gives the same log-decay on every channel."""
    rng = np.random.default_rng(5)
    a = rng.standard_normal((6, 3))
    _, _, g, _ = oracle.prepare_inputs(rng.standard_normal((6, 3, 4)), rng.standard_normal((6, 3, 4)),
                                       gate_logits=a, beta_logits=a, gate="scalar")
    for c in range(4):
        assert np.array_equal(g[..., c], g[..., 0])
    assert g[2, 1, 3] == pytest.approx(math.log(1.0 / (1.0 + math.exp(-a[2, 1]))), rel=1e-14)


# ------------------------------------------------- affine maps of segments (context parallelism)

def test_segment_is_an_affine_map_of_its_incoming_state():
    """A segment acts on its incoming state as S_out = M S_in + B, with M the run of the
    segment with v = 0 from the identity (dk = dv) and B its run from the zero state; the
    maps of consecutive segments compose, so a sequence split into segments gives the final
    state of the unsplit run (the exchange step of context-parallel prefill)."""
    rng = np.random.default_rng(17)
    T, H, d, P = 48, 2, 8, 3
    p = workloads.random_problem(rng, T, H, d, d)
    s0 = rng.standard_normal((1, H, d, d))
    _, s_ref = oracle.run(p["q"], p["k"], p["v"], p["g"], p["beta"], np.array([0, T], np.int32),
                          s0=s0)
    bounds = [0, 11, 30, T]
    eye = np.broadcast_to(np.eye(d), (P, H, d, d)).copy()
    cu = np.array(bounds, np.int32)
    _, M = oracle.run(p["q"], p["k"], np.zeros_like(p["v"]), p["g"], p["beta"], cu, s0=eye)
    _, B = oracle.run(p["q"], p["k"], p["v"], p["g"], p["beta"], cu, s0=np.zeros((P, H, d, d)))
    s = s0[0]
    for i in range(P):
        s = M[i] @ s + B[i]
    np.testing.assert_allclose(s, s_ref[0], rtol=0, atol=1e-12 * np.abs(s_ref).max())
    # the same holds for the additive write
    _, s_ref = oracle.run(p["q"], p["k"], p["v"], p["g"], p["beta"], np.array([0, T], np.int32),
                          s0=s0, mode=oracle.MODE_ADDITIVE)
    _, M = oracle.run(p["q"], p["k"], np.zeros_like(p["v"]), p["g"], p["beta"], cu, s0=eye,
                      mode=oracle.MODE_ADDITIVE)
    _, B = oracle.run(p["q"], p["k"], p["v"], p["g"], p["beta"], cu, s0=np.zeros((P, H, d, d)),
                      mode=oracle.MODE_ADDITIVE)
    s = s0[0]
    for i in range(P):
        s = M[i] @ s + B[i]
    np.testing.assert_allclose(s, s_ref[0], rtol=0, atol=1e-12 * np.abs(s_ref).max())


# ---------------------------------------------------------------- gradients
# The pages stop at the forward pass, so the backward oracle is a derivation;
# it is pinned to finite differences of the forward oracle, and to closed forms
# of the gradient in the cases where the recurrence has one.

def _bwd_problem(seed, T, H, dk, dv, N_cu=None, gate=-0.3):
    rng = np.random.default_rng(seed)
    q, k = rng.standard_normal((T, H, dk)), rng.standard_normal((T, H, dk))
    g = gate * np.abs(rng.standard_normal((T, H, dk)))
    v = rng.standard_normal((T, H, dv))
    beta = rng.random((T, H))
    cu = np.array([0, T] if N_cu is None else N_cu, dtype=np.int32)
    N = len(cu) - 1
    s0 = rng.standard_normal((N, H, dk, dv))
    do = rng.standard_normal((T, H, dv))
    dsf = rng.standard_normal((N, H, dk, dv))
    return dict(q=q, k=k, v=v, g=g, beta=beta, cu=cu, s0=s0, do=do, dsf=dsf)


def _loss(p, mode, **over):
    a = dict(p, **over)
    o, s = oracle.run(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], s0=a["s0"], mode=mode)
    return float((o * a["do"]).sum() + (s * a["dsf"]).sum())


@pytest.mark.parametrize("mode", [oracle.MODE_DELTA, oracle.MODE_ADDITIVE])
def test_gradients_match_central_differences(mode):
    """Every input's gradient, entry by entry, against (L(x+h) - L(x-h)) / 2h."""
    p = _bwd_problem(3, 9, 2, 3, 4, N_cu=[0, 4, 4, 9])   # a zero-length sequence in the middle
    r = oracle.run_bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], p["do"], p["cu"], s0=p["s0"],
                       ds_final=p["dsf"], mode=mode)
    h = 1e-6
    for name, key in [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"),
                      ("s0", "ds0")]:
        x = p[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            fd[idx] = (_loss(p, mode, **{name: xp}) - _loss(p, mode, **{name: xm})) / (2 * h)
        assert np.abs(fd - r[key]).max() <= 1e-7 * max(1.0, np.abs(fd).max()), name
    if mode == oracle.MODE_ADDITIVE:
        assert not r["dbeta"].any()


def test_gradient_directional_derivative_across_checkpoints():
    """Longer ragged sequences (the backward recomputes states from copies taken
    every 64 tokens): <grad, d> equals the central difference along d."""
    p = _bwd_problem(4, 230, 2, 8, 6, N_cu=[0, 70, 200, 230], gate=-0.05)
    r = oracle.run_bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], p["do"], p["cu"], s0=p["s0"],
                       ds_final=p["dsf"])
    rng = np.random.default_rng(5)
    keys = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"), ("s0", "ds0")]
    d = {name: rng.standard_normal(p[name].shape) for name, _ in keys}
    h = 1e-5
    plus = {name: p[name] + h * d[name] for name, _ in keys}
    minus = {name: p[name] - h * d[name] for name, _ in keys}
    fd = (_loss(p, oracle.MODE_DELTA, **plus) - _loss(p, oracle.MODE_DELTA, **minus)) / (2 * h)
    an = sum(float((r[key] * d[name]).sum()) for name, key in keys)
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an))


def test_gradient_beta_zero_closed_form():
    """beta = 0 and q = 0: the state only fades, S_T = Diag(exp(sum g)) S0, so
    dS0 = Diag(exp(sum g)) dS_T, every token's dg = rowsum(dS_T * S_T), dq_t = S_t do_t
    (S_t the faded state), dk = dv = 0, and dbeta_t = (G_t^T k_t) . (v_t - S_a,t^T k_t) with the cotangent
    G_t = Diag(exp(sum_{s>t} g_s)) dS_T and the faded state S_a,t = Diag(exp(sum_{s<=t} g_s)) S0."""
    p = _bwd_problem(6, 12, 1, 4, 3)
    p["beta"][:] = 0.0
    p["q"][:] = 0.0
    r = oracle.run_bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], p["do"], p["cu"], s0=p["s0"],
                       ds_final=p["dsf"])
    g, S0, W = p["g"][:, 0], p["s0"][0, 0], p["dsf"][0, 0]
    tot = g.sum(axis=0)
    ST = np.exp(tot)[:, None] * S0
    np.testing.assert_allclose(r["ds0"][0, 0], np.exp(tot)[:, None] * W, rtol=1e-12)
    for t in range(12):
        np.testing.assert_allclose(r["dg"][t, 0], (W * ST).sum(axis=1), rtol=1e-12)
        G = np.exp(g[t + 1:].sum(axis=0))[:, None] * W
        Sa = np.exp(g[:t + 1].sum(axis=0))[:, None] * S0
        kt, vt = p["k"][t, 0], p["v"][t, 0]
        np.testing.assert_allclose(r["dbeta"][t, 0], (G.T @ kt) @ (vt - Sa.T @ kt), rtol=1e-10)
        np.testing.assert_allclose(r["dq"][t, 0], Sa @ p["do"][t, 0], rtol=1e-10)
    for key in ("dk", "dv"):
        assert np.abs(r[key]).max() <= 1e-12


def test_gradient_linear_attention_closed_form():
    """Additive write, no fade: o = tril(Q K^T) V + Q S0 and S_T = S0 + K^T V, so
    with P = tril(Q K^T): dV = P^T dO + K dS_T, dP = tril(dO V^T), dQ = dP K + dO S0^T,
    dK = dP^T Q + V dS_T^T, dS0 = Q^T dO + dS_T (explicit T x T matrices)."""
    p = _bwd_problem(7, 10, 1, 5, 3)
    p["g"][:] = 0.0
    r = oracle.run_bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], p["do"], p["cu"], s0=p["s0"],
                       ds_final=p["dsf"], mode=oracle.MODE_ADDITIVE)
    Q, K, V, dO = p["q"][:, 0], p["k"][:, 0], p["v"][:, 0], p["do"][:, 0]
    S0, dST = p["s0"][0, 0], p["dsf"][0, 0]
    mask = np.tril(np.ones((10, 10)))
    P = mask * (Q @ K.T)
    dP = mask * (dO @ V.T)
    np.testing.assert_allclose(r["dv"][:, 0], P.T @ dO + K @ dST, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["dq"][:, 0], dP @ K + dO @ S0.T, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["dk"][:, 0], dP.T @ Q + V @ dST.T, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["ds0"][0, 0], Q.T @ dO + dST, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("gate,additive,gate_min", [("channel", False, -np.inf),
                                                    ("channel", False, -2.0),
                                                    ("scalar", False, -1.5),
                                                    ("none", True, -np.inf)])
def test_preparation_gradients_match_central_differences(gate, additive, gate_min):
    """prepare_inputs then the recurrence, as a function of the raw projections: the chain
    rule of prepare_inputs_bwd applied to run_bwd equals central differences entry by entry
    (with the gate floor active on some entries where set)."""
    rng = np.random.default_rng(8)
    T, H, dk, dv = 6, 1, 3, 2
    raw = dict(q=rng.standard_normal((T, H, dk)), k=rng.standard_normal((T, H, dk)),
               v=rng.standard_normal((T, H, dv)),
               a=2.0 * rng.standard_normal((T, H, dk)) if gate == "channel"
               else 2.0 * rng.standard_normal((T, H)) if gate == "scalar" else None,
               b=None if additive else rng.standard_normal((T, H)))
    mode = oracle.MODE_ADDITIVE if additive else oracle.MODE_DELTA
    do, dsf = rng.standard_normal((T, H, dv)), rng.standard_normal((1, H, dk, dv))

    def loss(r):
        q, k, g, beta = oracle.prepare_inputs(r["q"], r["k"], r["a"], r["b"], gate_min, gate)
        o, s = oracle.run(q, k, r["v"], g, beta, mode=mode)
        return float((o * do).sum() + (s * dsf).sum())

    q, k, g, beta = oracle.prepare_inputs(raw["q"], raw["k"], raw["a"], raw["b"], gate_min, gate)
    if np.isfinite(gate_min):
        ls = np.minimum(raw["a"], 0) - np.log1p(np.exp(-np.abs(raw["a"])))
        assert (ls < gate_min).any() and (ls > gate_min).any()
    gr = oracle.run_bwd(q, k, raw["v"], g, beta, do, ds_final=dsf, mode=mode)
    dq_raw, dk_raw, dgl, dbl = oracle.prepare_inputs_bwd(raw["q"], raw["k"], raw["a"], raw["b"],
                                                         gate_min, gate, gr["dq"], gr["dk"],
                                                         gr["dg"], gr["dbeta"])
    an = dict(q=dq_raw, k=dk_raw, v=gr["dv"], a=dgl, b=dbl)
    h = 1e-6
    for name in ("q", "k", "v", "a", "b"):
        if raw[name] is None:
            assert an[name] is None
            continue
        fd = np.zeros_like(raw[name])
        for idx in np.ndindex(raw[name].shape):
            rp = {kk: (vv.copy() if vv is not None else None) for kk, vv in raw.items()}
            rm = {kk: (vv.copy() if vv is not None else None) for kk, vv in raw.items()}
            rp[name][idx] += h
            rm[name][idx] -= h
            fd[idx] = (loss(rp) - loss(rm)) / (2 * h)
        assert np.abs(fd - an[name]).max() <= 1e-6 * max(1.0, np.abs(fd).max()), name
