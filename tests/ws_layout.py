"""Decoder of the prefill workspace layout (fp16 factors for bf16 inputs, fp32 for fp32), for tests that compare the GPU's
per-chunk intermediates with the CPU chunkwise form. It mirrors the layout
documented in gated_delta_rule_41_amd/csrc/kda_common.h (the "split" k order
inside each 32-deep slice: k(g, j) = 16 (j >> 2) + 4 g + (j & 3))."""
from __future__ import annotations

import numpy as np
import torch

CH = 64


def kslot(g, j):
    return 16 * (j >> 2) + 4 * g + (j & 3)


# position p = 8 g + j inside a slice -> logical index
SPLIT = np.array([kslot(p >> 3, p & 7) for p in range(32)])


def chunk_capacity(N, T, have_cu):
    return (T + CH - 1) // CH if not have_cu else (T + (CH - 1) * N) // CH


def plan(NC, H, D, f32):
    """Array offsets and total size. U is fp32 on both paths; with 16-bit
    factors A_qk is two fp16 planes (hi, lo), the output is fused into the state
    recursion and the chunk-entry states / corrected values stay on chip (their
    arrays are empty)."""
    es = 4 if f32 else 2
    ch = NC * H
    sizes = [ch * CH * D * es, ch * D * CH * es, ch * CH * D * es, ch * CH * D * 4,
             ch * CH * CH * 4, ch * D * 4, ch * D * D * es if f32 else 0, ch * CH * D * es if f32 else 0]
    off, o = [], 0
    for s in sizes:
        off.append(o)
        o = (o + s + 255) // 256 * 256
    return off, o


def seq_table(ws: torch.Tensor, N, T, H, D, f32, have_cu=True) -> np.ndarray:
    """The sequence table at the end of the workspace: [N + 1][start, len,
    first chunk slot, chunk count] int32."""
    _, o = plan(chunk_capacity(N, T, have_cu), H, D, f32)
    raw = ws[o:o + (N + 1) * 16].cpu().numpy()
    return raw.view(np.int32).reshape(N + 1, 4).copy()


def frag_rows(x: np.ndarray, nsl: int) -> np.ndarray:
    """Fragment order [4 row blocks][nsl slices][64 lanes][8] (lane n + 16 g: row
    16 I + n, slots of group g) -> row-major [64][nsl][32] in the split order."""
    t = x.reshape(4, nsl, 4, 16, 8)  # I, s, g, n, j
    return t.transpose(0, 3, 1, 2, 4).reshape(CH, nsl, 32)


def _as_f(raw: np.ndarray, f32: bool) -> np.ndarray:
    """fp32 factors with fp32 inputs; fp16 factors with bf16 inputs."""
    if f32:
        return raw.view(np.float32).astype(np.float64)
    return raw.view(np.float16).astype(np.float64)


def decode(ws: torch.Tensor, N, T, H, D, f32, have_cu, gc, h):
    """Intermediates of chunk slot gc, head h as fp64 numpy arrays."""
    NC = chunk_capacity(N, T, have_cu)
    off, _ = plan(NC, H, D, f32)
    es = 4 if f32 else 2
    raw = ws.cpu().numpy()
    chh = gc * H + h
    NS, NCT = D // 32, D // 16

    def arr(i, n_el, es_=es, f=f32):
        b = off[i] + chh * n_el * es_
        return _as_f(raw[b:b + n_el * es_].copy(), f)

    out = {}
    if f32:
        qp = arr(0, CH * D).reshape(CH, NS, 32)
    else:
        qp = frag_rows(arr(0, CH * D), NS)
    out["Qp"] = np.zeros((CH, D))
    out["Qp"][:, (np.arange(NS)[:, None] * 32 + SPLIT[None, :]).ravel()] = qp.reshape(CH, -1)
    km = arr(1, D * CH).reshape(D, 2, 32)
    Km_T = np.zeros((D, CH))
    Km_T[:, (np.arange(2)[:, None] * 32 + SPLIT[None, :]).ravel()] = km.reshape(D, -1)
    out["Km"] = Km_T.T
    wn = arr(2, CH * D).reshape(CH, NS, 32)
    W = np.zeros((CH, D))
    W[:, (np.arange(NS)[:, None] * 32 + SPLIT[None, :]).ravel()] = -wn.reshape(CH, -1)
    out["W"] = W
    u = arr(3, CH * D, 4, True).reshape(NCT, 4, 64, 4)
    U = np.zeros((CH, D))
    for ct in range(NCT):
        for I in range(4):
            for l in range(64):
                n, g = l & 15, l >> 4
                for i in range(4):
                    U[16 * I + 4 * g + i, 16 * ct + n] = u[ct, I, l, i]
    out["U"] = U
    if f32:
        aq = arr(4, CH * CH).reshape(CH, 2, 32)
    else:  # hi plane + lo plane, each in fragment order
        planes = arr(4, 2 * CH * CH).reshape(2, CH * CH)
        aq = frag_rows(planes[0], 2) + frag_rows(planes[1], 2)
    A = np.zeros((CH, CH))
    A[:, (np.arange(2)[:, None] * 32 + SPLIT[None, :]).ravel()] = aq.reshape(CH, -1)
    out["Aqk"] = A
    b = off[5] + chh * D * 4
    out["gam"] = raw[b:b + D * 4].copy().view(np.float32).astype(np.float64)
    if not f32:
        return out
    hh = arr(6, D * D).reshape(NCT, NS, 64, 8)
    Hm = np.zeros((D, D))
    vn = arr(7, CH * D).reshape(NCT, 2, 64, 8)
    Vn = np.zeros((CH, D))
    for ct in range(NCT):
        for l in range(64):
            n, g = l & 15, l >> 4
            for j in range(8):
                for s in range(NS):
                    Hm[32 * s + kslot(g, j), 16 * ct + n] = hh[ct, s, l, j]
                for s in range(2):
                    Vn[32 * s + kslot(g, j), 16 * ct + n] = vn[ct, s, l, j]
    out["h"] = Hm
    out["Vn"] = Vn
    return out


def plan_dplr(NC, H, D):
    """Offsets of the general-DPLR workspace (16-bit factors): qp, km, am, wn,
    u, aqk, oh, gam."""
    ch = NC * H
    f = ch * CH * D * 2
    sizes = [f, ch * D * max(D, CH) * 2, f, f, f, ch * CH * CH * 2, f, ch * D * 4]
    off, o = [], 0
    for s in sizes:
        off.append(o)
        o = (o + s + 255) // 256 * 256
    return off, o


def _tiles(raw16: np.ndarray, D) -> np.ndarray:
    """[D/16][4][64 lanes][4] accumulator-order tiles -> [64, D]."""
    t = raw16.reshape(D // 16, 4, 64, 4)
    out = np.zeros((CH, D))
    for ct in range(D // 16):
        for I in range(4):
            for l in range(64):
                n, g = l & 15, l >> 4
                out[16 * I + 4 * g:16 * I + 4 * g + 4, 16 * ct + n] = t[ct, I, l]
    return out


def decode_dplr(ws: torch.Tensor, N, T, H, D, have_cu, gc, h):
    """General-DPLR intermediates of chunk slot gc, head h (fp64): Qp, KV (= K-^T V),
    Am, W (= W'), U (= U'), Aqa, Oh (= A_qk V), gam."""
    NC = chunk_capacity(N, T, have_cu)
    off, _ = plan_dplr(NC, H, D)
    raw = ws.cpu().numpy()
    chh = gc * H + h
    NS = D // 32

    def arr(i, n_el):
        b = off[i] + chh * n_el * 2
        return _as_f(raw[b:b + n_el * 2].copy(), False)

    def kv_tiles(x):  # [D/16 col tile][D/16 row tile][64 lanes][4] -> [D, D]
        t = x.reshape(D // 16, D // 16, 64, 4)
        out = np.zeros((D, D))
        for ct in range(D // 16):
            for rt in range(D // 16):
                for l in range(64):
                    n, g = l & 15, l >> 4
                    out[16 * rt + 4 * g:16 * rt + 4 * g + 4, 16 * ct + n] = t[ct, rt, l]
        return out

    def split_cols(x, nsl):  # [rows][nsl][32] split order -> [rows, 32 nsl]
        out = np.zeros((x.shape[0], 32 * nsl))
        out[:, (np.arange(nsl)[:, None] * 32 + SPLIT[None, :]).ravel()] = x.reshape(x.shape[0], -1)
        return out

    out = {"Qp": split_cols(arr(0, CH * D).reshape(CH, NS, 32), NS),
           "KV": kv_tiles(arr(1, D * max(D, CH))[:D * D]),
           "Am": split_cols(arr(2, D * CH).reshape(D, 2, 32), 2).T,
           "W": -split_cols(arr(3, CH * D).reshape(CH, NS, 32), NS),
           "U": -_tiles(arr(4, CH * D), D),
           "Aqa": split_cols(arr(5, CH * CH).reshape(CH, 2, 32), 2),
           "Oh": _tiles(arr(6, CH * D), D)}
    b = off[7] + chh * D * 4
    out["gam"] = raw[b:b + D * 4].copy().view(np.float32).astype(np.float64)
    return out


def bwd_chunk_head_bytes(D):
    """Backward workspace per chunk-head of a piece: the fp32 forward plan, the
    state-gradient chain's U, h and V_new, the region its added term and then
    the local kernel's scratch share, and the gated key products."""
    fwd = plan(1, 1, D, True)[1]
    chain = CH * D * 4 + D * D * 4 + CH * D * 4
    shared = max(2 * CH * D, D * D) * 4
    return fwd + chain + shared + CH * CH * 4


def bwd_bytes(N, T, H, D, piece, have_cu=True):
    """Workspace of kda_chunk_bwd when it runs in pieces of `piece` chunk slots:
    the per-piece arrays, one [H][D][D] fp32 state per piece when there is more
    than one, the sequence table."""
    NC = chunk_capacity(N, T, have_cu)
    npieces = -(-NC // piece) if NC else 1
    table = ((N + 1) * 16 + 255) // 256 * 256
    return piece * H * bwd_chunk_head_bytes(D) + (npieces * H * D * D * 4 if npieces > 1 else 0) + table
