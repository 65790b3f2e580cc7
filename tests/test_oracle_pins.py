"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test is chosen so that a plausible mistake in the oracle (a dropped term,
a wrong sign, decay applied after the correction, reading the state before the
write, a transposed state or output, a wrong gate axis, a broken hand-off
between sequences) fails at least one of them. None of them re-types the
oracle's loop: they use closed forms, hand-derived values, special cases that
reduce to earlier methods, invariants and a dense-matrix brute force.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_case(T, H, dk, dv, *, shift=0.0, unit_k=True, beta=None):
    q = _unit(rng.standard_normal((T, H, dk)))
    k = rng.standard_normal((T, H, dk))
    if unit_k:
        k = _unit(k)
    v = rng.standard_normal((T, H, dv))
    la = -np.logaddexp(0.0, rng.standard_normal((T, H, dk)) + shift)
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H)))) if beta is None else np.full((T, H), beta)
    return q, k, v, la, b


def test_hand_scalar_golden():
    """dk = dv = 1 worked by hand (tests/golden/hand_scalar.json)."""
    g = json.load(open(os.path.join(GOLDEN, "hand_scalar.json")))
    T = len(g["k"])
    sh = lambda a: np.asarray(a, dtype=np.float64).reshape(T, 1, 1)
    o, S, _ = oracle.recurrence(sh(g["q"]), sh(g["k"]), sh(g["v"]), np.log(sh(g["alpha"])),
                                np.asarray(g["beta"], dtype=np.float64).reshape(T, 1),
                                np.full((1, 1, 1, 1), g["S0"]))
    np.testing.assert_allclose(o[:, 0, 0], g["o"], atol=g["tol"], rtol=0)
    assert abs(S[0, 0, 0, 0] - g["S_final"]) <= g["tol"]


def test_hand_2x2_golden():
    """dk = dv = 2 worked by hand (tests/golden/hand_2x2.json): pins the decay
    axis (key channels), the order decay -> correction -> write -> read, and
    that the output is S^T q rather than S q."""
    g = json.load(open(os.path.join(GOLDEN, "hand_2x2.json")))
    T = len(g["k"])
    a = lambda x: np.asarray(x, dtype=np.float64).reshape(T, 1, 2)
    o, S, _ = oracle.recurrence(a(g["q"]), a(g["k"]), a(g["v"]), np.log(a(g["alpha"])),
                                np.asarray(g["beta"], dtype=np.float64).reshape(T, 1),
                                np.asarray(g["S0"], dtype=np.float64).reshape(1, 1, 2, 2))
    np.testing.assert_allclose(o[:, 0, :], g["o"], atol=g["tol"], rtol=0)
    np.testing.assert_allclose(S[0, 0], g["S_final"], atol=g["tol"], rtol=0)


@pytest.mark.parametrize("shift", [0.0, 2.0, -2.0])
def test_exact_retrieval(shift):
    """With beta = 1 and unit keys, S_t^T k_t = v_t for any gates and any
    history (the delta rule's projection makes the new association exact), so
    with q = k the output equals v at every step."""
    T, H, dk, dv = 50, 3, 8, 5
    q, k, v, la, b = rand_case(T, H, dk, dv, shift=shift, beta=1.0)
    S0 = rng.standard_normal((1, H, dk, dv))
    o, _, _ = oracle.recurrence(k, k, v, la, b, S0)
    np.testing.assert_allclose(o, v, atol=1e-12, rtol=0)


def test_one_step_retrieval():
    """One step with beta = 1, alpha = 1 and unit k from any state: S^T k = v."""
    dk = dv = 16
    k = _unit(rng.standard_normal((1, 1, dk)))
    v = rng.standard_normal((1, 1, dv))
    o, S, _ = oracle.recurrence(k, k, v, np.zeros((1, 1, dk)), np.ones((1, 1)),
                                rng.standard_normal((1, 1, dk, dv)))
    np.testing.assert_allclose(S[0, 0].T @ k[0, 0], v[0, 0], atol=1e-12)


def test_beta_zero_closed_form():
    """beta = 0 leaves only the gates: o_t = S0^T (exp(G_t) * q_t) and
    S_T = Diag(exp(G_T)) S0, with G the inclusive cumulative log-gate."""
    T, H, dk, dv = 40, 2, 6, 7
    q, k, v, la, _ = rand_case(T, H, dk, dv, shift=-1.0)
    b = np.zeros((T, H))
    S0 = rng.standard_normal((1, H, dk, dv))
    o, S, _ = oracle.recurrence(q, k, v, la, b, S0)
    G = np.cumsum(la, axis=0)
    for h in range(H):
        exp_o = np.einsum("cj,tc->tj", S0[0, h], np.exp(G[:, h]) * q[:, h])
        np.testing.assert_allclose(o[:, h], exp_o, atol=1e-12, rtol=1e-12)
        np.testing.assert_allclose(S[0, h], np.exp(G[-1, h])[:, None] * S0[0, h], atol=1e-13)


def test_deltanet_reduction():
    """alpha = 1 reduces KDA to DeltaNet: S <- S + beta k (v - S^T k)^T
    (online gradient step on the reconstruction loss ||S^T k - v||^2 / 2)."""
    T, H, dk, dv = 30, 2, 5, 4
    q, k, v, _, b = rand_case(T, H, dk, dv)
    la = np.zeros((T, H, dk))
    S0 = rng.standard_normal((1, H, dk, dv))
    o, S, _ = oracle.recurrence(q, k, v, la, b, S0)
    for h in range(H):
        St = S0[0, h].copy()
        for t in range(T):
            grad = np.outer(k[t, h], St.T @ k[t, h] - v[t, h])  # d/dS of the loss
            St = St - b[t, h] * grad
            np.testing.assert_allclose(o[t, h], St.T @ q[t, h], atol=1e-12)
        np.testing.assert_allclose(S[0, h], St, atol=1e-12)


def test_gated_deltanet_reduction():
    """A gate constant across channels reduces KDA to Gated DeltaNet:
    S <- alpha (I - beta k k^T) S + beta k v^T."""
    T, H, dk, dv = 30, 2, 6, 3
    q, k, v, _, b = rand_case(T, H, dk, dv)
    a_scalar = -np.logaddexp(0.0, rng.standard_normal((T, H)))
    la = np.repeat(a_scalar[:, :, None], dk, axis=2)
    S0 = rng.standard_normal((1, H, dk, dv))
    o, S, _ = oracle.recurrence(q, k, v, la, b, S0)
    I = np.eye(dk)
    for h in range(H):
        St = S0[0, h].copy()
        for t in range(T):
            St = math.exp(a_scalar[t, h]) * (I - b[t, h] * np.outer(k[t, h], k[t, h])) @ St \
                + b[t, h] * np.outer(k[t, h], v[t, h])
            np.testing.assert_allclose(o[t, h], St.T @ q[t, h], atol=1e-12)
        np.testing.assert_allclose(S[0, h], St, atol=1e-12)


def test_dense_transition_brute_force():
    """Materialise the dense transition A_t = (I - beta k k^T) Diag(alpha) and
    run S_t = A_t S_{t-1} + beta k v^T with plain matrix products; keys are not
    normalised here, so nothing relies on ||k|| = 1."""
    T, H, dk, dv = 32, 2, 8, 8
    q, k, v, la, b = rand_case(T, H, dk, dv, unit_k=False)
    k *= 0.4
    S0 = rng.standard_normal((1, H, dk, dv))
    o, S, _ = oracle.recurrence(q, k, v, la, b, S0)
    for h in range(H):
        St = S0[0, h].copy()
        for t in range(T):
            A = (np.eye(dk) - b[t, h] * np.outer(k[t, h], k[t, h])) @ np.diag(np.exp(la[t, h]))
            St = A @ St + b[t, h] * np.outer(k[t, h], v[t, h])
            np.testing.assert_allclose(o[t, h], St.T @ q[t, h], atol=1e-12)
        np.testing.assert_allclose(S[0, h], St, atol=1e-12)


def test_householder_reflection_preserves_norm():
    """With beta = 2, alpha = 1, v = 0 and unit k, each step applies the
    Householder reflection I - 2 k k^T, which is orthogonal: ||S||_F is kept."""
    T, dk, dv = 25, 7, 5
    q, k, _, _, _ = rand_case(T, 1, dk, dv)
    S0 = rng.standard_normal((1, 1, dk, dv))
    _, S, _ = oracle.recurrence(q, k, np.zeros((T, 1, dv)), np.zeros((T, 1, dk)),
                                np.full((T, 1), 2.0), S0)
    assert abs(np.linalg.norm(S) - np.linalg.norm(S0)) < 1e-12


def test_linearity_in_values_and_state():
    """For fixed q, k, gates and beta, (V, S0) -> (O, S_T) is linear."""
    T, H, dk, dv = 20, 2, 6, 4
    q, k, v1, la, b = rand_case(T, H, dk, dv)
    v2 = rng.standard_normal(v1.shape)
    s1 = rng.standard_normal((1, H, dk, dv))
    s2 = rng.standard_normal((1, H, dk, dv))
    c1, c2 = 0.7, -1.3
    o1, S1, _ = oracle.recurrence(q, k, v1, la, b, s1)
    o2, S2, _ = oracle.recurrence(q, k, v2, la, b, s2)
    o3, S3, _ = oracle.recurrence(q, k, c1 * v1 + c2 * v2, la, b, c1 * s1 + c2 * s2)
    np.testing.assert_allclose(o3, c1 * o1 + c2 * o2, atol=1e-12)
    np.testing.assert_allclose(S3, c1 * S1 + c2 * S2, atol=1e-12)


def test_norm_bound_per_step():
    """||k|| = 1, beta in [0,1], alpha <= 1: (I - beta k k^T) Diag(alpha) has
    spectral norm <= 1 (its eigen-structure: 1 and 1 - beta for unit k), so
    ||S_t||_2 <= ||S_{t-1}||_2 + beta ||v_t||."""
    T, dk, dv = 40, 8, 6
    q, k, v, la, b = rand_case(T, 1, dk, dv, shift=-2.0)
    S = rng.standard_normal((1, 1, dk, dv)) * 3
    for t in range(T):
        sl = slice(t, t + 1)
        _, S_new, _ = oracle.recurrence(q[sl], k[sl], v[sl], la[sl], b[sl], S)
        lhs = np.linalg.norm(S_new[0, 0], 2)
        rhs = np.linalg.norm(S[0, 0], 2) + b[t, 0] * np.linalg.norm(v[t, 0])
        assert lhs <= rhs + 1e-12
        S = S_new


def test_split_and_carry_equals_whole():
    """A sequence run in pieces, each starting from the previous piece's final
    state, equals the whole run (the chunk hand-off)."""
    T, H, dk, dv = 70, 2, 5, 6
    q, k, v, la, b = rand_case(T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dk, dv))
    o, S, _ = oracle.recurrence(q, k, v, la, b, S0)
    Sc = S0
    parts = []
    for a, e in [(0, 1), (1, 17), (17, 64), (64, 70)]:
        sl = slice(a, e)
        op, Sc, _ = oracle.recurrence(q[sl], k[sl], v[sl], la[sl], b[sl], Sc)
        parts.append(op)
    np.testing.assert_array_equal(np.concatenate(parts), o)
    np.testing.assert_array_equal(Sc, S)


def test_varlen_pack_equals_separate():
    """A packed batch equals each sequence run alone, and a zero-length
    sequence returns its initial state."""
    lens = [5, 0, 33, 1, 12]
    T, H, dk, dv = sum(lens), 2, 4, 3
    q, k, v, la, b = rand_case(T, H, dk, dv)
    S0 = rng.standard_normal((len(lens), H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, S, _ = oracle.recurrence(q, k, v, la, b, S0, cu)
    for i, L in enumerate(lens):
        sl = slice(cu[i], cu[i + 1])
        oi, Si, _ = oracle.recurrence(q[sl], k[sl], v[sl], la[sl], b[sl], S0[i:i + 1])
        np.testing.assert_array_equal(o[sl], oi)
        np.testing.assert_array_equal(S[i], Si[0])
    np.testing.assert_array_equal(S[1], S0[1])


def test_prefill_then_decode_equals_longer_prefill():
    T, H, dk, dv = 19, 2, 4, 4
    q, k, v, la, b = rand_case(T + 1, H, dk, dv)
    S0 = rng.standard_normal((1, H, dk, dv))
    o_all, S_all, _ = oracle.recurrence(q, k, v, la, b, S0)
    _, S_T, _ = oracle.recurrence(q[:T], k[:T], v[:T], la[:T], b[:T], S0)
    od, Sd = oracle.decode_step(q[T:], k[T:], v[T:], la[T:], b[T:], S_T)
    np.testing.assert_array_equal(od[0], o_all[T])
    np.testing.assert_array_equal(Sd, S_all)


def test_bf16_inputs_are_read_exactly():
    """bf16 inputs are widened exactly: same result as the same values in fp64."""
    import torch
    T, H, dk, dv = 9, 2, 4, 4
    arrs = rand_case(T, H, dk, dv)
    tb = [torch.tensor(a).to(torch.bfloat16) for a in arrs]
    o1, S1, _ = oracle.recurrence(*tb)
    o2, S2, _ = oracle.recurrence(*[t.to(torch.float64) for t in tb])
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


def test_head_subset_column_blocks_and_recorded_positions():
    """Splitting value columns across threads, taking a subset of heads and
    recording sampled positions changes no arithmetic (bitwise equal)."""
    lens = [40, 25]
    T, H, dk, dv = sum(lens), 4, 6, 10
    q, k, v, la, b = rand_case(T, H, dk, dv)
    S0 = rng.standard_normal((2, H, dk, dv))
    cu = [0, 40, 65]
    o, S, _ = oracle.recurrence(q, k, v, la, b, S0, cu)
    heads = [3, 1]
    pos = [0, 7, 39, 40, 41, 64]
    o2, S2, orec = oracle.recurrence(q, k, v, la, b, S0, cu, heads=heads, rec_pos=pos,
                                     col_blocks=3, threads=3)
    for i, h in enumerate(heads):
        np.testing.assert_array_equal(o2[:, h], o[:, h])
        np.testing.assert_array_equal(S2[:, h], S[:, h])
        np.testing.assert_array_equal(orec[:, i], o[pos, h])
    assert not np.any(o2[:, 0])


def test_nan_propagates():
    T, H, dk, dv = 4, 1, 3, 3
    q, k, v, la, b = rand_case(T, H, dk, dv)
    v[1, 0, 2] = np.nan
    o, S, _ = oracle.recurrence(q, k, v, la, b)
    assert np.isnan(o[1:, 0, 2]).all()
    assert np.isfinite(o[0]).all()


def test_rejects_malformed_cu_seqlens():
    T, H, dk, dv = 6, 1, 2, 2
    q, k, v, la, b = rand_case(T, H, dk, dv)
    with pytest.raises(ValueError):
        oracle.recurrence(q, k, v, la, b, None, [0, 4, 3, 6])
    with pytest.raises(ValueError):
        oracle.recurrence(q, k, v, la, b, None, [0, 5])
