"""Pins of the layer prologue/epilogue oracle (oracle/layer.py) against library
routines, closed forms and special cases (CPU)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import layer as ly

rng = np.random.default_rng(5)


def test_conv_delta_filters():
    """A filter on the last tap is the identity; on the first tap it shifts the
    sequence by three rows, with zeros where the shift reaches before the start."""
    T, H, d = 11, 2, 5
    x = rng.standard_normal((T, H, d))
    w = np.zeros((H, d, 4))
    w[..., 3] = 1.0
    np.testing.assert_array_equal(ly.short_conv(x, w), x)
    w = np.zeros((H, d, 4))
    w[..., 0] = 1.0
    y = ly.short_conv(x, w)
    np.testing.assert_array_equal(y[3:], x[:-3])
    np.testing.assert_array_equal(y[:3], 0.0)


def test_conv_matches_library_per_sequence():
    """torch's grouped conv1d with left padding 3 is the same causal depthwise
    filter; packed sequences are convolved each from zero history."""
    lens = [7, 1, 0, 12]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, d = int(cu[-1]), 3, 4
    x = rng.standard_normal((T, H, d))
    w = rng.standard_normal((H, d, 4))
    got = ly.short_conv(x, w, cu)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        if a == b:
            continue
        xs = torch.from_numpy(x[a:b]).permute(1, 2, 0).reshape(1, H * d, b - a)   # [1, H*d, L]
        ws = torch.from_numpy(w).reshape(H * d, 1, 4)
        ref = F.conv1d(F.pad(xs, (3, 0)), ws, groups=H * d).reshape(H, d, b - a).permute(2, 0, 1)
        np.testing.assert_allclose(got[a:b], ref.numpy(), rtol=0, atol=1e-12)


def test_swish_sigmoid_softplus_match_library():
    x = np.concatenate([rng.standard_normal(200) * 8, [0.0, -80.0, 80.0]])
    t = torch.from_numpy(x)
    np.testing.assert_allclose(ly.swish(x), F.silu(t).numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(ly.sigmoid(x), torch.sigmoid(t).numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(ly.softplus(x), F.softplus(t).numpy(), rtol=1e-14, atol=1e-300)


def test_l2norm_unit_and_scale_free():
    x = rng.standard_normal((6, 2, 16))
    n = np.linalg.norm(ly.l2norm(x), axis=-1)
    np.testing.assert_allclose(n, 1.0, atol=1e-6)
    np.testing.assert_allclose(ly.l2norm(1000.0 * x), ly.l2norm(x), rtol=1e-7)  # up to eps


def test_decay_gate_closed_forms():
    # A_log = 0 and dt_bias = 0 at a = 0: log alpha = -log 2
    la = ly.decay_gate(np.zeros((1, 1, 3)), np.zeros(1), np.zeros((1, 3)))
    np.testing.assert_allclose(la, -np.log(2.0), rtol=1e-15)
    # scaling by exp(A_log) per head, the bias per channel
    a = rng.standard_normal((4, 2, 3))
    A_log = np.array([0.5, -1.0])
    dtb = rng.standard_normal((2, 3))
    ref = -np.exp(A_log)[None, :, None] * np.log1p(np.exp(a + dtb[None]))
    np.testing.assert_allclose(ly.decay_gate(a, A_log, dtb), ref, rtol=1e-13)
    assert np.all(ly.decay_gate(a, A_log, dtb) < 0)


def test_epilogue_matches_library_rms_norm():
    o = rng.standard_normal((5, 2, 8))
    g = rng.standard_normal((5, 2, 8))
    w = rng.standard_normal(8)
    ref = F.rms_norm(torch.from_numpy(o), (8,), torch.from_numpy(w), eps=ly.EPS) * torch.sigmoid(torch.from_numpy(g))
    np.testing.assert_allclose(ly.layer_epilogue(o, g, w), ref.numpy(), rtol=1e-12)


def test_epilogue_constant_row():
    """A constant row c normalises to c / sqrt(c^2 + eps); a zero gate
    pre-activation halves it."""
    o = np.full((1, 1, 4), 3.0)
    y = ly.layer_epilogue(o, np.zeros((1, 1, 4)), np.ones(4))
    np.testing.assert_allclose(y, 0.5 * 3.0 / np.sqrt(9.0 + ly.EPS), rtol=1e-15)


def test_prologue_outputs_are_valid_operator_inputs():
    """q and k come out unit-norm, log alpha negative, beta in (0, 1), and the
    convolution never reaches into the previous sequence."""
    lens = [5, 9]
    cu = np.array([0, 5, 14])
    T, H, d = 14, 2, 8
    xs = [rng.standard_normal((T, H, d)) for _ in range(4)]
    xb = rng.standard_normal((T, H))
    ws = [rng.standard_normal((H, d, 4)) for _ in range(3)]
    q, k, v, la, b = ly.layer_prologue(*xs, xb, *ws, rng.standard_normal(H), rng.standard_normal((H, d)), cu)
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 1.0, atol=1e-5)
    np.testing.assert_allclose(np.linalg.norm(k, axis=-1), 1.0, atol=1e-5)
    assert np.all(la < 0) and np.all((b > 0) & (b < 1))
    # the second sequence's first value row sees only its own first pre-activation row
    ref = ly.swish(ws[2][:, :, 3] * xs[2][5])
    np.testing.assert_allclose(v[5], ref, rtol=1e-13)


@pytest.mark.parametrize("L", [0, 1, 2, 3, 9])
def test_decode_prologue_continues_the_prefill(L):
    """The history after L tokens plus the prologue of token L in decode form
    equals the prefill prologue's row L over L + 1 tokens, and the shifted
    history equals the history after L + 1 tokens (lengths below the filter's
    width included: the history starts as zeros)."""
    H, d = 2, 6
    x = [rng.standard_normal((L + 1, H, d)) for _ in range(4)]
    xb = rng.standard_normal((L + 1, H))
    w = [rng.standard_normal((H, d, 4)) for _ in range(3)]
    A_log, dtb = rng.standard_normal(H), rng.standard_normal((H, d))
    full = ly.layer_prologue(*x, xb, *w, A_log, dtb)
    st = ly.conv_state(x[0][:L], x[1][:L], x[2][:L])
    got = ly.layer_decode_prologue(x[0][L:], x[1][L:], x[2][L:], x[3][L:], xb[L:], st, *w, A_log, dtb)
    for a, b in zip(got[:5], full):
        np.testing.assert_allclose(a, b[L:], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(got[5], ly.conv_state(x[0], x[1], x[2]))


def test_conv_state_packed_and_short():
    """Per sequence, oldest row first; an empty sequence's history is zero, a
    one-token sequence's is (0, 0, x_0)."""
    lens = [5, 0, 1]
    cu = np.array([0, 5, 5, 6])
    x = [rng.standard_normal((6, 1, 3)) for _ in range(3)]
    st = ly.conv_state(*x, cu)
    assert st.shape == (3, 1, 3, 3, 3)
    for m in range(3):
        np.testing.assert_array_equal(st[0, :, m], np.moveaxis(x[m][2:5], 0, 1))
        np.testing.assert_array_equal(st[2, :, m, 2], x[m][5])
    np.testing.assert_array_equal(st[1], 0.0)
    np.testing.assert_array_equal(st[2, :, :, :2], 0.0)
