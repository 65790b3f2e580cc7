"""Chunkwise-parallel form of the KDA recurrence, fp64 numpy -- TEST INFRASTRUCTURE.

A second witness beside the token recurrence in ``kda_oracle.c``, written
separately from it and sharing no code with the HIP path. It follows the
chunkwise algorithm the pages describe in prose (GeekNews "Kimi Linear"
summary, sections "Algoritmo paralelo por chunks" and "Menos computação que o
DPLR geral"):

* the sequence is cut into fixed-size chunks and each chunk starts from the
  previous chunk's final state;
* the chunk's rank-1 updates are gathered in a WY representation: one
  triangular inverse T = (I + A_kk)^-1 (the UT transform) serves both factors
  W = T Diag(beta) K+ and U = T Diag(beta) V, and nothing downstream inverts
  again;
* that unit-lower-triangular inverse is built row by row by forward
  substitution;
* the state update is in matrix form per chunk, and the output adds an
  inter-chunk (recurrent) part to an intra-chunk (parallel) part;
* because the DPLR transition ties both of its low-rank vectors to the key,
  only two gated intra-chunk matrices are needed: A_kk and A_qk.

Derivation (from the recurrence, per chunk of L tokens, local index r):
  g_r = sum_{s<=r} log alpha_s              (per key channel, inclusive)
  K+_r = exp(g_r) * k_r,  Q+_r = exp(g_r) * q_r,  K-_r = exp(g_{L-1} - g_r) * k_r
  A_kk[r,i] = beta_r sum_c k_rc k_ic exp(g_rc - g_ic)        (i < r)
  A_qk[r,i] = sum_c q_rc k_ic exp(g_rc - g_ic)               (i <= r)
  T = (I + A_kk)^-1;  W = T Diag(beta) K+;  U = T Diag(beta) V
  V_new = U - W S;  O = Q+ S + A_qk V_new
  S <- Diag(exp(g_{L-1})) S + K-^T V_new

Options reproduce two numerical devices of the GPU path so that their algebra
is pinned in fp64 against the recurrence:
  ``sub``      secondary chunking of the gated products: the exponentials are
               anchored at sub-chunk starts, exp(g_r - g_i) =
               exp(g_r - g_a(I)) * exp(g_a(I) - g_a(J)) * exp(g_a(J) - g_i),
               so every factor stays bounded (the log-domain precision issue
               the pages raise for divisions inside a chunk);
  ``blocked``  the UT transform applied by blocked forward substitution on the
               right-hand sides, X_I = T_II (B_I - sum_{K<I} A_IK X_K), with
               the diagonal blocks T_II inverted row by row.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def _f64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def forward_substitution_inverse(A: np.ndarray) -> np.ndarray:
    """Inverse of the unit lower-triangular matrix I + A (A strictly lower),
    built row by row: T[r, :r] = -A[r, :r] @ T[:r, :r], T[r, r] = 1."""
    n = A.shape[0]
    T = np.eye(n)
    for r in range(1, n):
        T[r, :r] = -A[r, :r] @ T[:r, :r]
    return T


def gated_products(x, y, g, sub: Optional[int] = None, strict: bool = False):
    """P[r, i] = sum_c x_rc y_ic exp(g_rc - g_ic) for i <= r (i < r if strict), else 0."""
    L = x.shape[0]
    P = np.zeros((L, L))
    if sub is None:
        for r in range(L):
            top = r if strict else r + 1
            if top == 0:
                continue
            P[r, :top] = (x[r][None, :] * y[:top] * np.exp(g[r][None, :] - g[:top])).sum(axis=1)
        return P
    nb = (L + sub - 1) // sub
    for I in range(nb):
        rI = slice(I * sub, min(L, (I + 1) * sub))
        aI = I * sub
        E = np.exp(g[rI] - g[aI])              # <= 1
        for J in range(I + 1):
            rJ = slice(J * sub, min(L, (J + 1) * sub))
            aJ = J * sub
            c = np.exp(g[aI] - g[aJ])          # <= 1
            Einv = np.exp(g[aJ] - g[rJ])       # >= 1, bounded by the sub-chunk's range
            blk = (x[rI] * E * c) @ (y[rJ] * Einv).T
            if I == J:
                n = blk.shape[0]
                mask = np.tril(np.ones((n, n)), -1 if strict else 0)
                blk = blk * mask
            P[rI, rJ] = blk
    return P


def blocked_solve(A: np.ndarray, B: np.ndarray, sub: int) -> np.ndarray:
    """Solve (I + A) X = B by blocked forward substitution with diagonal-block inverses."""
    L = A.shape[0]
    X = np.zeros_like(B)
    nb = (L + sub - 1) // sub
    for I in range(nb):
        rI = slice(I * sub, min(L, (I + 1) * sub))
        Y = B[rI].copy()
        for K in range(I):
            rK = slice(K * sub, min(L, (K + 1) * sub))
            Y -= A[rI, rK] @ X[rK]
        X[rI] = forward_substitution_inverse(A[rI, rI]) @ Y
    return X


def chunk_step(q, k, v, la, b, S, *, sub=None, blocked=None):
    """One chunk: returns (O, S_next, intermediates dict)."""
    L = q.shape[0]
    g = np.cumsum(la, axis=0)
    Kp = np.exp(g) * k
    Qp = np.exp(g) * q
    Km = np.exp(g[L - 1][None, :] - g) * k
    gam = np.exp(g[L - 1])
    Akk = b[:, None] * gated_products(k, k, g, sub=sub, strict=True)
    Aqk = gated_products(q, k, g, sub=sub, strict=False)
    rhs = np.concatenate([b[:, None] * Kp, b[:, None] * v], axis=1)
    if blocked:
        X = blocked_solve(Akk, rhs, blocked)
    else:
        T = forward_substitution_inverse(Akk)
        X = T @ rhs
    dk = k.shape[1]
    W, U = X[:, :dk], X[:, dk:]
    Vn = U - W @ S
    O = Qp @ S + Aqk @ Vn
    S_next = gam[:, None] * S + Km.T @ Vn
    inter = dict(g=g, Qp=Qp, Km=Km, Kp=Kp, gam=gam, Akk=Akk, Aqk=Aqk, W=W, U=U, Vn=Vn, h=S.copy())
    return O, S_next, inter


def chunkwise(q, k, v, log_alpha, beta, initial_state=None, cu_seqlens=None, *,
              chunk: int = 64, sub: Optional[int] = None, blocked: Optional[int] = None,
              heads: Optional[Sequence[int]] = None, keep: bool = False):
    """Chunkwise fp64 forward over a packed batch. Same shapes and return
    convention as ``oracle.recurrence`` (o, S_final); with ``keep`` a third
    item lists per-(sequence, head, chunk) intermediates."""
    q, k, v, la, b = (_f64(x) for x in (q, k, v, log_alpha, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = [0, T] if cu_seqlens is None else [int(x) for x in _f64(cu_seqlens)]
    N = len(cu) - 1
    S0 = None if initial_state is None else _f64(initial_state)
    o = np.zeros((T, H, dv))
    S_fin = np.zeros((N, H, dk, dv))
    kept = []
    hs = range(H) if heads is None else heads
    for n in range(N):
        for h in hs:
            S = np.zeros((dk, dv)) if S0 is None else S0[n, h].copy()
            for c0 in range(cu[n], cu[n + 1], chunk):
                c1 = min(c0 + chunk, cu[n + 1])
                sl = slice(c0, c1)
                O, S, inter = chunk_step(q[sl, h], k[sl, h], v[sl, h], la[sl, h], b[sl, h], S,
                                         sub=sub, blocked=blocked)
                o[sl, h] = O
                if keep:
                    kept.append(((n, h, c0), inter))
            S_fin[n, h] = S
    if keep:
        return o, S_fin, kept
    return o, S_fin


# ---------------------------------------------------------------------------
# General DPLR transition, chunkwise (the comparison operator)
#
#   S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t
#
# KDA ties both low-rank vectors to the key; with free a and b the chunk needs
# four gated intra-chunk matrices instead of two (GeekNews "Kimi Linear"
# summary, section "Menos computação que o DPLR geral"). Derivation, per chunk
# of L tokens with entry state H, inclusive cumulative log-gate g_r and
# exclusive one e_r = g_r - log alpha_r (the low-rank read of row r sees the
# state before row r's decay):
#   u_r = S_{r-1}^T b_r = H^T (b_r exp(e_r)) + sum_{s<r} A_bk[r,s] v_s - sum_{s<r} A_ba[r,s] u_s
#   A_bx[r,s] = sum_c b_rc x_sc exp(e_rc - g_sc)   (s < r)
#   A_qx[r,s] = sum_c q_rc x_sc exp(g_rc - g_sc)   (s <= r)
#   so u = W' H + U' with T = (I + A_ba)^-1, W' = T B~ (B~_r = exp(e_r) b_r), U' = T A_bk V;
#   O  = Q+ H + A_qk V - A_qa u
#   S' = Diag(exp(g_last)) H + K-^T V - A-^T u   (K-, A-: rows scaled by exp(g_last - g_s))
# ---------------------------------------------------------------------------


def gated_products_lr(x, gl, y, gr, e, sub: Optional[int] = None, strict: bool = False):
    """P[r, i] = sum_c x_rc y_ic exp(gl_rc - gr_ic) for i <= r (i < r if strict).

    With ``sub`` the exponentials are anchored at the exclusive gate e at each
    sub-chunk start a (e_a = gate total before the sub-chunk):
    exp(gl_r - gr_i) = exp(gl_r - e_aI) exp(e_aI - e_aJ) exp(e_aJ - gr_i);
    for gl in {g, e} and gr = g the first two factors are <= 1 and the last lies
    in [1, exp(-sum of log alpha over sub-chunk J)]."""
    L = x.shape[0]
    P = np.zeros((L, L))
    if sub is None:
        for r in range(L):
            top = r if strict else r + 1
            if top == 0:
                continue
            P[r, :top] = (x[r][None, :] * y[:top] * np.exp(gl[r][None, :] - gr[:top])).sum(axis=1)
        return P
    nb = (L + sub - 1) // sub
    for I in range(nb):
        rI = slice(I * sub, min(L, (I + 1) * sub))
        eI = e[I * sub]
        left = x[rI] * np.exp(gl[rI] - eI)
        for J in range(I + 1):
            rJ = slice(J * sub, min(L, (J + 1) * sub))
            eJ = e[J * sub]
            blk = (left * np.exp(eI - eJ)) @ (y[rJ] * np.exp(eJ - gr[rJ])).T
            if I == J:
                n = blk.shape[0]
                blk = blk * np.tril(np.ones((n, n)), -1 if strict else 0)
            P[rI, rJ] = blk
    return P


def dplr_chunk_step(q, k, v, a, b, la, S, *, sub=None, blocked=None):
    """One DPLR chunk: returns (O, S_next, intermediates dict)."""
    L = q.shape[0]
    g = np.cumsum(la, axis=0)
    e = g - la
    Qp = np.exp(g) * q
    Bt = np.exp(e) * b
    dec = np.exp(g[L - 1][None, :] - g)
    Km, Am = dec * k, dec * a
    gam = np.exp(g[L - 1])
    Aba = gated_products_lr(b, e, a, g, e, sub=sub, strict=True)
    Abk = gated_products_lr(b, e, k, g, e, sub=sub, strict=True)
    Aqk = gated_products_lr(q, g, k, g, e, sub=sub, strict=False)
    Aqa = gated_products_lr(q, g, a, g, e, sub=sub, strict=False)
    rhs = np.concatenate([Bt, Abk @ v], axis=1)
    if blocked:
        X = blocked_solve(Aba, rhs, blocked)
    else:
        X = forward_substitution_inverse(Aba) @ rhs
    dk = k.shape[1]
    W, U = X[:, :dk], X[:, dk:]
    u = W @ S + U
    Oh = Aqk @ v
    O = Qp @ S + Oh - Aqa @ u
    S_next = gam[:, None] * S + Km.T @ v - Am.T @ u
    inter = dict(g=g, Qp=Qp, Km=Km, Am=Am, Bt=Bt, gam=gam, Aba=Aba, Abk=Abk, Aqk=Aqk, Aqa=Aqa,
                 W=W, U=U, u=u, Oh=Oh, KV=Km.T @ v, h=S.copy())
    return O, S_next, inter


def dplr_chunkwise(q, k, v, a, b, log_alpha, initial_state=None, cu_seqlens=None, *,
                   chunk: int = 64, sub: Optional[int] = None, blocked: Optional[int] = None,
                   keep: bool = False):
    """Chunkwise fp64 forward of the general DPLR transition over a packed
    batch; same shapes and return convention as ``oracle.dplr_recurrence``."""
    q, k, v, a, b, la = (_f64(x) for x in (q, k, v, a, b, log_alpha))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = [0, T] if cu_seqlens is None else [int(x) for x in _f64(cu_seqlens)]
    N = len(cu) - 1
    S0 = None if initial_state is None else _f64(initial_state)
    o = np.zeros((T, H, dv))
    S_fin = np.zeros((N, H, dk, dv))
    kept = []
    for n in range(N):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else S0[n, h].copy()
            for c0 in range(cu[n], cu[n + 1], chunk):
                sl = slice(c0, min(c0 + chunk, cu[n + 1]))
                O, S, inter = dplr_chunk_step(q[sl, h], k[sl, h], v[sl, h], a[sl, h], b[sl, h], la[sl, h], S,
                                              sub=sub, blocked=blocked)
                o[sl, h] = O
                if keep:
                    kept.append(((n, h, c0), inter))
            S_fin[n, h] = S
    if keep:
        return o, S_fin, kept
    return o, S_fin
