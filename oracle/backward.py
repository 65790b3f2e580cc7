"""Gradients of the KDA operator -- TEST INFRASTRUCTURE.

Only ``tests/`` and ``bench.py``'s CPU-baseline leg may import this module; the
product path never does.

* ``recurrence_grads`` -- the oracle: reverse-mode differentiation (torch
  autograd, fp64, CPU) of the plain token-by-token recurrence
      S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
      o_t = S_t^T q_t,  alpha_t = exp(log_alpha_t),
  written out step by step below (GeekNews "Kimi Linear" summary, sections
  "Da atenção linear ao Gated DeltaNet" and "Controle fino de memória no Kimi
  Delta Attention"; the chunkwise algorithm is presented there as a training
  algorithm, section "Algoritmo paralelo por chunks", which needs these
  gradients). Given upstream gradients dO of o and dS of the final states, it
  returns dq, dk, dv, dlog_alpha, dbeta and the gradient of the initial states.
  Pinned by central finite differences in ``tests/test_backward_cpu.py``.
* ``chunkwise_grads`` -- a separately written fp64 numpy witness: the backward
  of the chunkwise form (reverse chunk recursion for the state gradient, the
  chunk-local adjoints of the output, of the WY/UT factors and of the gated
  products, and a reverse cumulative sum for the gate), which the GPU backward
  follows. Checked against the oracle to 1e-10.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _t64(x):
    import torch
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64)
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


def recurrence_grads(q, k, v, log_alpha, beta, initial_state=None, cu_seqlens=None, d_o=None,
                     d_final=None):
    """Token-loop fp64 autograd. Shapes as ``oracle.recurrence``; d_o [T, H, dv]
    (None = zeros), d_final [N, H, dk, dv] (None = zeros). Returns a dict of
    numpy fp64 arrays: dq, dk, dv, dlog_alpha, dbeta, dinitial_state, plus the
    forward o and final states."""
    import torch
    q, k, v, la, b = (_t64(x).clone().requires_grad_(True) for x in (q, k, v, log_alpha, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = [0, T] if cu_seqlens is None else [int(x) for x in np.asarray(_t64(cu_seqlens))]
    N = len(cu) - 1
    S0 = torch.zeros(N, H, dk, dv, dtype=torch.float64) if initial_state is None else _t64(initial_state).clone()
    S0.requires_grad_(True)
    outs, finals = [], []
    for n in range(N):
        S = S0[n]  # [H, dk, dv]
        for t in range(cu[n], cu[n + 1]):
            alpha = torch.exp(la[t])                                   # [H, dk]
            S = alpha[:, :, None] * S                                  # decay
            u = b[t][:, None] * (v[t] - torch.einsum("hcj,hc->hj", S, k[t]))  # residual vs the decayed state
            S = S + k[t][:, :, None] * u[:, None, :]                   # write
            outs.append(torch.einsum("hcj,hc->hj", S, q[t]))           # read the updated state
        finals.append(S)
    o = torch.stack(outs) if outs else torch.zeros(0, H, dv, dtype=torch.float64)
    Sf = torch.stack(finals)
    gO = torch.zeros_like(o) if d_o is None else _t64(d_o)
    gS = torch.zeros_like(Sf) if d_final is None else _t64(d_final)
    loss = (o * gO).sum() + (Sf * gS).sum()
    grads = torch.autograd.grad(loss, [q, k, v, la, b, S0], allow_unused=True)
    names = ["dq", "dk", "dv", "dlog_alpha", "dbeta", "dinitial_state"]
    out = {}
    for nm, g, ref in zip(names, grads, [q, k, v, la, b, S0]):
        out[nm] = (torch.zeros_like(ref) if g is None else g).detach().numpy()
    out["o"] = o.detach().numpy()
    out["final_state"] = Sf.detach().numpy()
    return out


# ---------------------------------------------------------------------------
# chunkwise witness
# ---------------------------------------------------------------------------

def _fwd_chunk(q, k, v, la, b, S):
    """Forward of one chunk, keeping what the backward needs."""
    L = q.shape[0]
    g = np.cumsum(la, axis=0)
    E = np.exp(g)
    Kp, Qp = E * k, E * q
    Km = np.exp(g[L - 1][None, :] - g) * k
    gam = np.exp(g[L - 1])
    # gated products with their exponent matrices (rows r, cols i, channels c)
    D = np.exp(np.clip(g[:, None, :] - g[None, :, :], None, 0.0))  # exp(g_r - g_i), only i <= r is used
    Pkk = np.einsum("rc,ic,ric->ri", k, k, D) * np.tril(np.ones((L, L)), -1)
    Pqk = np.einsum("rc,ic,ric->ri", q, k, D) * np.tril(np.ones((L, L)), 0)
    Akk = b[:, None] * Pkk
    Tm = np.linalg.inv(np.eye(L) + Akk)
    B = np.concatenate([b[:, None] * Kp, b[:, None] * v], axis=1)
    X = Tm @ B
    dk = k.shape[1]
    W, U = X[:, :dk], X[:, dk:]
    Vn = U - W @ S
    O = Qp @ S + Pqk @ Vn
    S_next = gam[:, None] * S + Km.T @ Vn
    return O, S_next, dict(g=g, E=E, Kp=Kp, Qp=Qp, Km=Km, gam=gam, D=D, Pkk=Pkk, Pqk=Pqk, Tm=Tm, B=B,
                           W=W, U=U, Vn=Vn, h=S.copy())


def _bwd_chunk(q, k, v, la, b, c, dO, dS_next):
    """Backward of one chunk given the gradient of its exit state; returns
    (dq, dk, dv, dla, db, dS_entry)."""
    L, dk = q.shape
    h, Vn, W, Tm, B = c["h"], c["Vn"], c["W"], c["Tm"], c["B"]
    # output and state update
    dVn = c["Pqk"].T @ dO + c["Km"] @ dS_next
    dQp = dO @ h.T
    dPqk = (dO @ Vn.T) * np.tril(np.ones((L, L)), 0)
    dKm = Vn @ dS_next.T
    dgam = (h * dS_next).sum(axis=1)
    dW = -dVn @ h.T
    dU = dVn
    dS_entry = c["gam"][:, None] * dS_next + c["Qp"].T @ dO - W.T @ dVn
    # UT transform: X = T B, T = (I + A_kk)^-1
    dX = np.concatenate([dW, dU], axis=1)
    dB = Tm.T @ dX
    dTm = dX @ B.T
    dAkk = -(Tm.T @ dTm @ Tm.T) * np.tril(np.ones((L, L)), -1)
    dBk, dBv = dB[:, :dk], dB[:, dk:]
    dbeta = (c["Kp"] * dBk).sum(axis=1) + (v * dBv).sum(axis=1) + (dAkk * c["Pkk"]).sum(axis=1)
    dKp = b[:, None] * dBk
    dv = b[:, None] * dBv
    dPkk = b[:, None] * dAkk
    # gated products P[r,i] = sum_c x_rc y_ic exp(g_rc - g_ic)
    D = c["D"]
    dq = np.einsum("ri,ic,ric->rc", dPqk, k, D)
    dk_ = np.einsum("ri,rc,ric->ic", dPqk, q, D)
    dk_ += np.einsum("ri,ic,ric->rc", dPkk, k, D) + np.einsum("ri,rc,ric->ic", dPkk, k, D)
    Gq = np.einsum("ri,rc,ic,ric->ric", dPqk, q, k, D)
    Gk = np.einsum("ri,rc,ic,ric->ric", dPkk, k, k, D)
    dg = Gq.sum(axis=1) - Gq.sum(axis=0) + Gk.sum(axis=1) - Gk.sum(axis=0)
    # gated scalings
    E = c["E"]
    dq += E * dQp
    dg += dQp * c["Qp"]
    dk_ += E * dKp
    dg += dKp * c["Kp"]
    dk_ += np.exp(c["g"][L - 1][None, :] - c["g"]) * dKm
    t = dKm * c["Km"]
    dg -= t
    dg[L - 1] += t.sum(axis=0) + dgam * c["gam"]
    # g = cumsum(log_alpha): reverse cumulative sum
    dla = np.cumsum(dg[::-1], axis=0)[::-1]
    return dq, dk_, dv, dla, dbeta, dS_entry


def chunkwise_grads(q, k, v, log_alpha, beta, initial_state=None, cu_seqlens=None, d_o=None,
                    d_final=None, *, chunk: int = 64):
    """Chunkwise fp64 backward (forward recomputed per chunk, then the reverse
    chunk recursion); same returns as ``recurrence_grads``."""
    f = lambda x: None if x is None else np.asarray(_t64(x).numpy(), dtype=np.float64)
    q, k, v, la, b = (f(x) for x in (q, k, v, log_alpha, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = [0, T] if cu_seqlens is None else [int(x) for x in np.asarray(_t64(cu_seqlens))]
    N = len(cu) - 1
    S0 = np.zeros((N, H, dk, dv)) if initial_state is None else f(initial_state)
    gO = np.zeros((T, H, dv)) if d_o is None else f(d_o)
    gS = np.zeros((N, H, dk, dv)) if d_final is None else f(d_final)
    out = {nm: np.zeros_like(x) for nm, x in
           (("dq", q), ("dk", k), ("dv", v), ("dlog_alpha", la), ("dbeta", b), ("dinitial_state", S0))}
    out["o"] = np.zeros((T, H, dv))
    out["final_state"] = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            S = S0[n, h].copy()
            saved = []
            for c0 in range(cu[n], cu[n + 1], chunk):
                sl = slice(c0, min(c0 + chunk, cu[n + 1]))
                O, S, c = _fwd_chunk(q[sl, h], k[sl, h], v[sl, h], la[sl, h], b[sl, h], S)
                out["o"][sl, h] = O
                saved.append((sl, c))
            out["final_state"][n, h] = S
            dS = gS[n, h].copy()
            for sl, c in reversed(saved):
                dq, dk_, dv_, dla, db, dS = _bwd_chunk(q[sl, h], k[sl, h], v[sl, h], la[sl, h], b[sl, h], c,
                                                       gO[sl, h], dS)
                out["dq"][sl, h] = dq
                out["dk"][sl, h] = dk_
                out["dv"][sl, h] = dv_
                out["dlog_alpha"][sl, h] = dla
                out["dbeta"][sl, h] = db
            out["dinitial_state"][n, h] = dS
    return out
