"""The KDA layer's prologue and epilogue around the operator -- TEST INFRASTRUCTURE.

Only ``tests/`` and ``bench.py``'s CPU-baseline leg may import this module; the
product path never does.

The GeekNews "Kimi Linear" summary, section "Configuração do modelo Kimi
Linear", describes what surrounds the operator in a KDA layer: the query, key
and value of every head pass through a short convolution and Swish; the query
and key are L2-normalised; the per-channel decay gate comes from a low-rank
projection through a decay function like GDN's and Mamba's; and before the
output projection a per-head RMSNorm and a data-dependent output gate are
applied. The projections themselves (matrix products with trained weights)
are model matters and are not here: these functions start from their outputs
(the pre-activations) and end before the output projection.

Where the page leaves a detail open, the plainest reading is taken:
* short convolution: causal, depthwise (one filter per head and channel),
  width 4, no bias, zero history before each sequence's first token (the
  convolution never crosses a sequence boundary);
* Swish: x * sigmoid(x);
* L2 norm over the head dimension, x / sqrt(sum x^2 + eps), eps = 1e-6;
* decay gate: log alpha = -exp(A_log[h]) * softplus(a + dt_bias[h, c]), the
  Mamba-style form GDN also uses, with one A_log per head and one dt_bias per
  key channel;
* beta = sigmoid(b), one per token and head;
* output: RMSNorm over the head's value dimension with a weight per value
  channel, o / sqrt(mean o^2 + eps) * w, eps = 1e-6, times the output gate
  sigmoid(g), g the gate's pre-activation per value channel.

Everything is fp64 numpy, written step by step from these definitions.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

CONV_WIDTH = 4
EPS = 1e-6


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _bounds(T: int, cu_seqlens) -> list:
    return [0, T] if cu_seqlens is None else [int(v) for v in np.asarray(_f64(cu_seqlens))]


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def softplus(x):
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def short_conv(x, w, cu_seqlens=None):
    """Causal depthwise convolution: y[t, h, c] = sum_i w[h, c, i] x[t - 3 + i, h, c],
    with x = 0 before the first token of t's sequence. x [T, H, d], w [H, d, 4]."""
    x, w = _f64(x), _f64(w)
    T = x.shape[0]
    y = np.zeros_like(x)
    b = _bounds(T, cu_seqlens)
    for n in range(len(b) - 1):
        for t in range(b[n], b[n + 1]):
            for i in range(CONV_WIDTH):
                s = t - (CONV_WIDTH - 1) + i
                if s >= b[n]:
                    y[t] += w[:, :, i] * x[s]
    return y


def swish(x):
    x = _f64(x)
    return x * sigmoid(x)


def l2norm(x):
    x = _f64(x)
    return x / np.sqrt((x * x).sum(axis=-1, keepdims=True) + EPS)


def decay_gate(a, A_log, dt_bias):
    """log alpha [T, H, dk] from the gate pre-activation a [T, H, dk], A_log [H],
    dt_bias [H, dk]."""
    a, A_log, dt_bias = _f64(a), _f64(A_log), _f64(dt_bias)
    return -np.exp(A_log)[None, :, None] * softplus(a + dt_bias[None])


def layer_prologue(xq, xk, xv, xa, xb, wq, wk, wv, A_log, dt_bias, cu_seqlens=None):
    """Pre-activations -> the operator's inputs (q, k, v, log_alpha, beta), fp64."""
    q = l2norm(swish(short_conv(xq, wq, cu_seqlens)))
    k = l2norm(swish(short_conv(xk, wk, cu_seqlens)))
    v = swish(short_conv(xv, wv, cu_seqlens))
    return q, k, v, decay_gate(xa, A_log, dt_bias), sigmoid(_f64(xb))


def conv_state(xq, xk, xv, cu_seqlens=None):
    """The convolution's history after each sequence, for one-token decoding: the
    last CONV_WIDTH - 1 rows of xq, xk, xv, oldest first, with zero rows where
    the sequence is shorter. Returns [N, H, 3 (q, k, v), CONV_WIDTH - 1, d]."""
    xs = [_f64(x) for x in (xq, xk, xv)]
    T, H, d = xs[0].shape
    b = _bounds(T, cu_seqlens)
    out = np.zeros((len(b) - 1, H, 3, CONV_WIDTH - 1, d))
    for n in range(len(b) - 1):
        for i in range(CONV_WIDTH - 1):
            t = b[n + 1] - (CONV_WIDTH - 1) + i
            if t >= b[n]:
                for m in range(3):
                    out[n, :, m, i] = xs[m][t]
    return out


def layer_decode_prologue(xq, xk, xv, xa, xb, state, wq, wk, wv, A_log, dt_bias):
    """One token per sequence (xq, xk, xv, xa [N, H, d], xb [N, H]) after the
    history ``state`` [N, H, 3, CONV_WIDTH - 1, d]: the convolution reads the
    history's rows and then the new one. Returns (q, k, v, log_alpha, beta,
    the history shifted by the new row)."""
    state = _f64(state)
    new = [_f64(x) for x in (xq, xk, xv)]
    ws = [_f64(w) for w in (wq, wk, wv)]
    y = []
    for m in range(3):
        win = np.concatenate([state[:, :, m], new[m][:, :, None]], axis=2)  # [N, H, 4, d]
        acc = np.zeros_like(new[m])
        for i in range(CONV_WIDTH):
            acc += ws[m][None, :, :, i] * win[:, :, i]
        y.append(acc)
    q = l2norm(swish(y[0]))
    k = l2norm(swish(y[1]))
    v = swish(y[2])
    nxt = np.concatenate([state[:, :, :, 1:], np.stack(new, axis=2)[:, :, :, None]], axis=3)
    return q, k, v, decay_gate(xa, A_log, dt_bias), sigmoid(_f64(xb)), nxt


def layer_epilogue(o, g, rms_w):
    """The operator's output o [T, H, dv] -> RMSNorm(o) * rms_w * sigmoid(g), fp64."""
    o, g, rms_w = _f64(o), _f64(g), _f64(rms_w)
    rms = np.sqrt((o * o).mean(axis=-1, keepdims=True) + EPS)
    return o / rms * rms_w * sigmoid(g)


def layer(xq, xk, xv, xa, xb, xg, wq, wk, wv, A_log, dt_bias, rms_w, initial_state=None,
          cu_seqlens=None, round_inputs_to=None):
    """The whole layer between the projections: prologue, the operator (the C
    oracle's recurrence) and epilogue. ``round_inputs_to`` (a torch dtype) rounds
    the operator's inputs as a caller storing them in that dtype would."""
    import oracle
    q, k, v, la, b = layer_prologue(xq, xk, xv, xa, xb, wq, wk, wv, A_log, dt_bias, cu_seqlens)
    if round_inputs_to is not None:
        import torch
        q, k, v, la, b = (torch.from_numpy(x).to(round_inputs_to).double().numpy() for x in (q, k, v, la, b))
    o, S, _ = oracle.recurrence(q, k, v, la, b, initial_state, cu_seqlens)
    return layer_epilogue(o, xg, rms_w), S, (q, k, v, la, b, o)
