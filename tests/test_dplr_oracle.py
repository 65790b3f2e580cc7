"""Pins of the general-DPLR oracle (``oracle.dplr_recurrence``) against facts
fixed by mathematics and by the KDA oracle it must specialise to.

The transition S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T is the
general diagonal-plus-low-rank form that KDA ties to the key (GeekNews "Kimi
Linear" summary, section "Menos computação que o DPLR geral"). A plausible
mistake in the loop (decay applied before the low-rank read, a wrong sign on
a u^T, a and b swapped, the write key dropped, a broken hand-off between
sequences) fails at least one of: the hand-derived example, the reduction to
the (separately pinned) KDA oracle, exact retrieval, the closed forms with
a = 0 (masked linear attention, gated linear attention) and the
varlen/separate equivalence.
"""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(4321)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def test_hand_2x2_golden():
    """dk = dv = 2 worked by hand (tests/golden/dplr_hand_2x2.json)."""
    g = json.load(open(os.path.join(GOLDEN, "dplr_hand_2x2.json")))
    arr = lambda key: np.array(g[key], dtype=np.float64)[:, None, :]  # [T, H=1, d]
    la = np.log(arr("alpha"))
    S0 = np.array(g["S0"], dtype=np.float64)[None, None]
    o, S = oracle.dplr_recurrence(arr("q"), arr("k"), arr("v"), arr("a"), arr("b"), la, S0)
    np.testing.assert_allclose(o[:, 0], np.array(g["o"]), rtol=0, atol=g["tol"])
    np.testing.assert_allclose(S[0, 0], np.array(g["S_final"]), rtol=0, atol=g["tol"])


def test_reduces_to_kda():
    """a = beta k, b = alpha * k and written key beta k give the KDA transition
    (I - beta k k^T) Diag(alpha) S + beta k v^T, whose oracle is pinned on its own."""
    T, H, dk, dv = 150, 2, 8, 6
    cu = np.array([0, 37, 37, 150])
    q = _unit(rng.standard_normal((T, H, dk)))
    k = _unit(rng.standard_normal((T, H, dk)))
    v = rng.standard_normal((T, H, dv))
    la = -np.logaddexp(0.0, rng.standard_normal((T, H, dk)) - 1.0)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    S0 = rng.standard_normal((3, H, dk, dv))
    o_k, S_k, _ = oracle.recurrence(q, k, v, la, beta, S0, cu)
    bk = beta[..., None] * k
    o_d, S_d = oracle.dplr_recurrence(q, bk, v, bk, np.exp(la) * k, la, S0, cu)
    scale = max(np.abs(o_k).max(), 1.0)
    assert np.abs(o_d - o_k).max() < 1e-11 * scale
    assert np.abs(S_d - S_k).max() < 1e-11 * max(np.abs(S_k).max(), 1.0)


def test_exact_retrieval():
    """With a = k (unit), b = alpha * k and q = k the transition is
    (I - k k^T) Diag(alpha) S + k v^T, so S_t^T k_t = v_t exactly for any gate
    and any earlier state: the read must see the state before the token and
    the decay must act between the read and the write."""
    T, H, dk, dv = 40, 3, 5, 4
    k = _unit(rng.standard_normal((T, H, dk)))
    v = rng.standard_normal((T, H, dv))
    la = -np.abs(rng.standard_normal((T, H, dk)))
    S0 = rng.standard_normal((1, H, dk, dv))
    o, _ = oracle.dplr_recurrence(k, k, v, k, np.exp(la) * k, la, S0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)


def test_masked_linear_attention():
    """a = 0 and alpha = 1: o = tril(Q K^T) V + Q S0 and S_final = S0 + K^T V
    (causal linear attention, computed with library matrix products)."""
    T, H, dk, dv = 33, 2, 6, 5
    q, k, a, b = (rng.standard_normal((T, H, dk)) for _ in range(4))
    v = rng.standard_normal((T, H, dv))
    S0 = rng.standard_normal((1, H, dk, dv))
    o, S = oracle.dplr_recurrence(q, k, v, np.zeros_like(a), b, np.zeros((T, H, dk)), S0)
    for h in range(H):
        Q, K, V = q[:, h], k[:, h], v[:, h]
        ref = np.tril(Q @ K.T) @ V + Q @ S0[0, h]
        np.testing.assert_allclose(o[:, h], ref, rtol=0, atol=1e-10)
        np.testing.assert_allclose(S[0, h], S0[0, h] + K.T @ V, rtol=0, atol=1e-10)


def test_gated_linear_attention_closed_form():
    """a = 0 with a channel-wise gate: the unrolled closed form
    o_t = sum_{s<=t} (sum_c q_tc k_sc exp(G_tc - G_sc)) v_s + (exp(G_t) * q_t)^T S0,
    G the inclusive cumulative log-gate; b must then have no effect."""
    T, H, dk, dv = 25, 1, 4, 3
    q, k, b = (rng.standard_normal((T, H, dk)) for _ in range(3))
    v = rng.standard_normal((T, H, dv))
    la = -np.abs(rng.standard_normal((T, H, dk)))
    S0 = rng.standard_normal((1, H, dk, dv))
    o, S = oracle.dplr_recurrence(q, k, v, np.zeros((T, H, dk)), b, la, S0)
    G = np.cumsum(la[:, 0], axis=0)
    ref = np.zeros((T, dv))
    for t in range(T):
        for s in range(t + 1):
            ref[t] += (q[t, 0] * k[s, 0] * np.exp(G[t] - G[s])).sum() * v[s, 0]
        ref[t] += (np.exp(G[t]) * q[t, 0]) @ S0[0, 0]
    np.testing.assert_allclose(o[:, 0], ref, rtol=0, atol=1e-10)
    S_ref = np.exp(G[-1])[:, None] * S0[0, 0] + sum(
        np.outer(np.exp(G[-1] - G[s]) * k[s, 0], v[s, 0]) for s in range(T))
    np.testing.assert_allclose(S[0, 0], S_ref, rtol=0, atol=1e-10)


def test_varlen_pack_equals_separate_and_column_blocks():
    """Sequences packed with cu_seqlens run independently, each from its own
    initial state; splitting the value columns over workers changes nothing."""
    lens = [5, 0, 17, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, dk, dv = int(cu[-1]), 2, 4, 6
    q, k, a, b = (rng.standard_normal((T, H, dk)) * 0.5 for _ in range(4))
    v = rng.standard_normal((T, H, dv))
    la = -np.abs(rng.standard_normal((T, H, dk)))
    S0 = rng.standard_normal((len(lens), H, dk, dv))
    o, S = oracle.dplr_recurrence(q, k, v, a, b, la, S0, cu, col_blocks=3)
    for i in range(len(lens)):
        sl = slice(cu[i], cu[i + 1])
        o1, S1 = oracle.dplr_recurrence(q[sl], k[sl], v[sl], a[sl], b[sl], la[sl], S0[i:i + 1])
        np.testing.assert_array_equal(o[sl], o1)
        np.testing.assert_array_equal(S[i], S1[0])


def test_bf16_inputs_are_read_exactly():
    """bf16 inputs (raw 16-bit patterns) are widened exactly: the result equals
    the fp64 run on the same rounded values."""
    import torch
    T, H, d = 20, 1, 8
    x = [torch.randn(T, H, d).to(torch.bfloat16) for _ in range(5)]
    la = -torch.rand(T, H, d).to(torch.bfloat16)
    o16, S16 = oracle.dplr_recurrence(*x, la)
    o64, S64 = oracle.dplr_recurrence(*[t.double() for t in x], la.double())
    np.testing.assert_array_equal(o16, o64)
    np.testing.assert_array_equal(S16, S64)
