"""The CPU chunkwise form (fp64) against the token recurrence, and its pieces
against textbook routines. Agreement to 1e-10 over many chunk sizes, partial
chunks and packed batches pins the chunk algebra (WY/UT factors, the two
gated intra-chunk matrices, the inter-chunk state recursion) that the GPU
kernels implement, including the anchored secondary chunking of the gated
products and the blocked forward substitution."""
import numpy as np
import pytest

import oracle
from oracle import chunkwise as cw

rng = np.random.default_rng(77)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def case(T, H, dk, dv, shift=0.0):
    q = _unit(rng.standard_normal((T, H, dk)))
    k = _unit(rng.standard_normal((T, H, dk)))
    v = rng.standard_normal((T, H, dv))
    la = -np.logaddexp(0.0, rng.standard_normal((T, H, dk)) + shift)
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, la, b


def _err(a, b):
    return np.max(np.abs(a - b)) / max(np.sqrt(np.mean(b * b)), 1e-300)


@pytest.mark.parametrize("T", [1, 5, 63, 64, 65, 200])
@pytest.mark.parametrize("chunk", [1, 2, 4, 16, 64])
def test_chunkwise_matches_recurrence(T, chunk):
    H, dk, dv = 2, 8, 4
    q, k, v, la, b = case(T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dk, dv))
    o_ref, S_ref, _ = oracle.recurrence(q, k, v, la, b, S0)
    o, S = cw.chunkwise(q, k, v, la, b, S0, chunk=chunk)
    assert _err(o, o_ref) <= 1e-10
    assert _err(S, S_ref) <= 1e-10


@pytest.mark.parametrize("dims", [(4, 4), (8, 8), (64, 64), (16, 8)])
@pytest.mark.parametrize("sub,blocked", [(None, None), (4, None), (16, None), (16, 16), (None, 4)])
def test_secondary_chunking_and_blocked_solve(dims, sub, blocked):
    dk, dv = dims
    T, H = 150, 1
    q, k, v, la, b = case(T, H, dk, dv, shift=1.0)
    S0 = rng.standard_normal((1, H, dk, dv))
    o_ref, S_ref, _ = oracle.recurrence(q, k, v, la, b, S0)
    o, S = cw.chunkwise(q, k, v, la, b, S0, chunk=64, sub=sub, blocked=blocked)
    assert _err(o, o_ref) <= 1e-10
    assert _err(S, S_ref) <= 1e-10


def test_fast_decay_secondary_chunking():
    """Per-chunk decay far beyond exp(-88) (fp32 overflow of the naive
    factorisation) is still exact with anchored sub-chunks."""
    T, H, dk, dv = 128, 1, 8, 8
    q, k, v, _, b = case(T, H, dk, dv)
    la = -np.abs(rng.standard_normal((T, H, dk))) * 6.0
    o_ref, S_ref, _ = oracle.recurrence(q, k, v, la, b)
    o, S = cw.chunkwise(q, k, v, la, b, chunk=64, sub=16, blocked=16)
    assert _err(o, o_ref) <= 1e-10
    assert _err(S, S_ref) <= 1e-10


def test_varlen_chunkwise():
    lens = [1, 64, 0, 130, 17]
    T, H, dk, dv = sum(lens), 2, 8, 8
    q, k, v, la, b = case(T, H, dk, dv)
    S0 = rng.standard_normal((len(lens), H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o_ref, S_ref, _ = oracle.recurrence(q, k, v, la, b, S0, cu)
    o, S = cw.chunkwise(q, k, v, la, b, S0, cu, chunk=64, sub=16, blocked=16)
    assert _err(o, o_ref) <= 1e-10
    assert _err(S, S_ref) <= 1e-10


def test_forward_substitution_against_library_solve():
    for n in [1, 2, 16, 64]:
        A = np.tril(rng.standard_normal((n, n)) * 0.3, -1)
        T = cw.forward_substitution_inverse(A)
        I = np.eye(n)
        np.testing.assert_allclose(T @ (I + A), I, atol=1e-13)
        np.testing.assert_allclose(T, np.linalg.solve(I + A, I), atol=1e-12)


def test_gated_products_definition():
    """Secondary chunking returns the same matrix as the elementwise definition."""
    L, d = 64, 8
    x = rng.standard_normal((L, d))
    y = rng.standard_normal((L, d))
    g = np.cumsum(-np.abs(rng.standard_normal((L, d))), axis=0)
    brute = np.zeros((L, L))
    for r in range(L):
        for i in range(r + 1):
            brute[r, i] = sum(x[r, c] * y[i, c] * np.exp(g[r, c] - g[i, c]) for c in range(d))
    np.testing.assert_allclose(cw.gated_products(x, y, g), brute, atol=1e-12)
    np.testing.assert_allclose(cw.gated_products(x, y, g, sub=16), brute, atol=1e-12)
    strict = cw.gated_products(x, y, g, sub=16, strict=True)
    np.testing.assert_allclose(strict, np.tril(brute, -1), atol=1e-12)


def test_padding_rows_are_neutral():
    """Rows with k = q = v = 0, beta = 0, log_alpha = 0 appended to a chunk
    change neither the outputs of the real rows nor the carried state."""
    T, dk, dv = 40, 8, 8
    q, k, v, la, b = case(T, 1, dk, dv)
    S0 = rng.standard_normal((dk, dv))
    O1, S1, _ = cw.chunk_step(q[:, 0], k[:, 0], v[:, 0], la[:, 0], b[:, 0], S0)
    pad = lambda a: np.concatenate([a, np.zeros((24,) + a.shape[1:])])
    O2, S2, _ = cw.chunk_step(pad(q[:, 0]), pad(k[:, 0]), pad(v[:, 0]), pad(la[:, 0]),
                              pad(b[:, 0]), S0, sub=16, blocked=16)
    np.testing.assert_allclose(O2[:T], O1, atol=1e-12)
    np.testing.assert_allclose(S2, S1, atol=1e-12)


def dplr_case(T, H, dk, dv, shift=0.0):
    q = _unit(rng.standard_normal((T, H, dk)))
    k = _unit(rng.standard_normal((T, H, dk)))
    v = rng.standard_normal((T, H, dv))
    ah = _unit(rng.standard_normal((T, H, dk)))
    la = -np.logaddexp(0.0, rng.standard_normal((T, H, dk)) + shift)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, beta[..., None] * ah, np.exp(la) * ah, la


@pytest.mark.parametrize("T", [1, 17, 64, 65, 200])
@pytest.mark.parametrize("chunk", [1, 4, 16, 64])
def test_dplr_chunkwise_matches_recurrence(T, chunk):
    """The four-matrix chunk algebra of the general DPLR transition (and its
    anchored secondary chunking / blocked substitution) equals the token loop."""
    H, dk, dv = 2, 8, 4
    q, k, v, a, b, la = dplr_case(T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dk, dv))
    o_ref, S_ref = oracle.dplr_recurrence(q, k, v, a, b, la, S0)
    o, S = cw.dplr_chunkwise(q, k, v, a, b, la, S0, chunk=chunk)
    assert _err(o, o_ref) < 1e-10 and _err(S, S_ref) < 1e-10
    if chunk >= 16:
        o2, S2 = cw.dplr_chunkwise(q, k, v, a, b, la, S0, chunk=chunk, sub=16, blocked=16)
        assert _err(o2, o_ref) < 1e-10 and _err(S2, S_ref) < 1e-10


def test_dplr_chunkwise_independent_ab_varlen_fast_decay():
    """Independent a and b (no structure shared with k), packed sequences and
    the fast-decay gate, with secondary chunking: still the token loop."""
    lens = [64, 1, 130, 0, 77]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, dk, dv = int(cu[-1]), 2, 16, 8
    q = _unit(rng.standard_normal((T, H, dk)))
    k = _unit(rng.standard_normal((T, H, dk)))
    a = 0.5 * _unit(rng.standard_normal((T, H, dk)))
    b = 0.5 * _unit(rng.standard_normal((T, H, dk)))
    v = rng.standard_normal((T, H, dv))
    la = -np.logaddexp(0.0, rng.standard_normal((T, H, dk)) + 2.0)
    S0 = rng.standard_normal((len(lens), H, dk, dv))
    o_ref, S_ref = oracle.dplr_recurrence(q, k, v, a, b, la, S0, cu)
    o, S = cw.dplr_chunkwise(q, k, v, a, b, la, S0, cu, sub=16, blocked=16)
    assert _err(o, o_ref) < 1e-10 and _err(S, S_ref) < 1e-10


def test_dplr_anchored_factors_are_bounded():
    """With the exclusive-gate anchors every left and cross factor is <= 1 and
    every right factor lies in [1, exp(-sum of log alpha over its sub-chunk)]."""
    L, dk, sub = 64, 8, 16
    la = -np.logaddexp(0.0, rng.standard_normal((L, dk)) + 2.0)
    g = np.cumsum(la, axis=0)
    e = g - la
    for I in range(L // sub):
        rI = slice(I * sub, (I + 1) * sub)
        eI = e[I * sub]
        assert np.all(g[rI] - eI <= 1e-12) and np.all(e[rI] - eI <= 1e-12)
        for J in range(I + 1):
            eJ = e[J * sub]
            assert np.all(eI - eJ <= 1e-12)
            right = eJ - g[J * sub:(J + 1) * sub]
            assert np.all(right >= -1e-12)
            assert np.all(right <= -la[J * sub:(J + 1) * sub].sum(axis=0) + 1e-12)
