"""The gradient oracle (fp64 autograd through the token recurrence) pinned by
central finite differences, and the chunkwise backward witness against it.

The finite differences perturb the inputs of the plain C recurrence (the
forward oracle, pinned on its own), so the gradient oracle is checked against
something other than itself: a wrong adjoint anywhere (the order of decay and
correction, the beta placement, the state hand-off between sequences) changes a
directional derivative."""
import numpy as np
import pytest

import oracle
from oracle import backward as bw

rng = np.random.default_rng(99)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def case(T, H, dk, dv, n_seq=1, shift=0.0):
    q = _unit(rng.standard_normal((T, H, dk)))
    k = _unit(rng.standard_normal((T, H, dk)))
    v = rng.standard_normal((T, H, dv))
    la = -np.logaddexp(0.0, rng.standard_normal((T, H, dk)) + shift)
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    S0 = rng.standard_normal((n_seq, H, dk, dv))
    return q, k, v, la, b, S0


def loss(inputs, cu, dO, dS):
    q, k, v, la, b, S0 = inputs
    o, S, _ = oracle.recurrence(q, k, v, la, b, S0, cu)
    return float((o * dO).sum() + (S * dS).sum())


@pytest.mark.parametrize("which", range(6))
def test_gradients_match_central_differences(which):
    """Directional derivative along a random direction, for each input in turn."""
    T, H, dk, dv = 23, 2, 5, 4
    cu = np.array([0, 9, 9, 23])
    inputs = list(case(T, H, dk, dv, n_seq=3))
    dO = rng.standard_normal((T, H, dv))
    dS = rng.standard_normal((3, H, dk, dv))
    g = bw.recurrence_grads(*inputs, cu, dO, dS)
    name = ["dq", "dk", "dv", "dlog_alpha", "dbeta", "dinitial_state"][which]
    direction = rng.standard_normal(inputs[which].shape)
    eps = 1e-6
    plus = [x.copy() for x in inputs]
    minus = [x.copy() for x in inputs]
    plus[which] = plus[which] + eps * direction
    minus[which] = minus[which] - eps * direction
    fd = (loss(plus, cu, dO, dS) - loss(minus, cu, dO, dS)) / (2 * eps)
    an = float((g[name] * direction).sum())
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_forward_of_the_gradient_oracle_is_the_oracle():
    T, H, dk, dv = 40, 2, 6, 3
    q, k, v, la, b, S0 = case(T, H, dk, dv)
    g = bw.recurrence_grads(q, k, v, la, b, S0, None, np.zeros((T, H, dv)), None)
    o, S, _ = oracle.recurrence(q, k, v, la, b, S0)
    np.testing.assert_allclose(g["o"], o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(g["final_state"], S, rtol=0, atol=1e-13)


@pytest.mark.parametrize("chunk", [1, 16, 64])
@pytest.mark.parametrize("shift", [-2.0, 2.0])
def test_chunkwise_backward_matches_oracle(chunk, shift):
    """The chunkwise backward (reverse chunk recursion for the state gradient,
    adjoints of the output, of the WY/UT factors and of the gated products, a
    reverse cumulative sum for the gate) equals the oracle on packed sequences
    with partial chunks and an empty sequence."""
    lens = [70, 0, 150, 5]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, dk, dv = int(cu[-1]), 2, 8, 6
    q, k, v, la, b, S0 = case(T, H, dk, dv, n_seq=len(lens), shift=shift)
    dO = rng.standard_normal((T, H, dv))
    dS = rng.standard_normal((len(lens), H, dk, dv))
    ref = bw.recurrence_grads(q, k, v, la, b, S0, cu, dO, dS)
    got = bw.chunkwise_grads(q, k, v, la, b, S0, cu, dO, dS, chunk=chunk)
    for name in ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dinitial_state", "o", "final_state"):
        scale = max(np.abs(ref[name]).max(), 1e-300)
        assert np.abs(got[name] - ref[name]).max() <= 1e-10 * scale, name
