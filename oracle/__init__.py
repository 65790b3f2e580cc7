"""CPU oracle for the KDA operator -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path (the HIP library behind
``include/kda.h`` and its Python binding) never imports, links or runs it, and
this package imports nothing from the product.

Contents
--------
* ``recurrence``  -- the oracle proper: the plain token-by-token fp64 recurrence
  (C, OpenMP over independent (sequence, head, column-block) units), see
  ``kda_oracle.c`` for the formula and its sources.
* ``chunkwise``   -- a second, separately written fp64 witness: the chunkwise
  parallel form (WY/UT factors, forward substitution, inter-chunk state
  recursion) derived from the same recurrence; it also serves as the spec of
  the chunk intermediates.
* ``dplr_recurrence`` -- the same kind of fp64 token loop for the general
  diagonal-plus-low-rank transition S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1}
  + k_t v_t^T that KDA specialises (the comparison operator).
* ``build``       -- compiles ``kda_oracle.c`` with the host C compiler.
* ``backward``    -- (module) the gradients: fp64 autograd through the recurrence.
* ``layer``       -- (module) the layer's prologue (short convolution, Swish,
  L2 norm, decay and beta gates) and epilogue (RMSNorm, output gate) around
  the operator, pinned by ``tests/test_layer_cpu.py``.

Pinned by ``tests/test_oracle_pins.py`` (exact retrieval, beta = 0 closed form,
DeltaNet and Gated DeltaNet reductions, dense-transition brute force,
linearity, norm bound, split/carry and varlen/separate equivalence, a
hand-derived scalar example in ``tests/golden``), ``tests/test_dplr_oracle.py``
(the DPLR loop against the KDA oracle, masked linear attention, exact
retrieval, a hand-derived example) and by
``tests/test_chunkwise_cpu.py`` (chunkwise form equal to the recurrence to
1e-10 in fp64; triangular inverse against a library solve).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
# the in-tree build; KDA_ORACLE_LIBRARY may name another build of kda_oracle.c
# (e.g. one with sanitizers)
_LIB_PATH = os.environ.get("KDA_ORACLE_LIBRARY") or os.path.join(_HERE, "libkda_oracle.so")
_lib = None

ORC_F32, ORC_BF16, ORC_F64 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the C oracle into ``oracle/libkda_oracle.so`` (portable x86-64-v3)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared",
               "-std=c11", "-Wall", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        f = lib.kda_oracle_forward
        f.restype = ctypes.c_int
        P = ctypes.c_void_p
        f.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                      P, P, P, P, P, ctypes.c_int, ctypes.c_int,
                      ctypes.c_int32, P, P, P, P, P, ctypes.c_int32, P, ctypes.c_int64, P,
                      ctypes.c_int32, ctypes.c_int32]
        f = lib.kda_oracle_dplr_forward
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                      P, P, P, P, P, P, ctypes.c_int, ctypes.c_int,
                      ctypes.c_int32, P, P, P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
        _lib = lib
    return _lib


def _as_host_buffer(x):
    """Return (contiguous numpy array holding the raw values, dtype code)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu").contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy(), ORC_BF16
            if x.dtype == torch.float32:
                return x.numpy(), ORC_F32
            if x.dtype == torch.float64:
                return x.numpy(), ORC_F64
            raise TypeError(f"unsupported dtype {x.dtype}")
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, ORC_F32
    if x.dtype == np.float64:
        return x, ORC_F64
    if x.dtype in (np.uint16, np.int16):
        return x, ORC_BF16
    raise TypeError(f"unsupported dtype {x.dtype}")


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def recurrence(q, k, v, log_alpha, beta, initial_state=None, cu_seqlens=None, *,
               heads: Optional[Sequence[int]] = None, want_o: bool = True,
               rec_pos: Optional[Sequence[int]] = None, col_blocks: int = 1,
               threads: int = 0):
    """Token-by-token fp64 KDA recurrence over a packed batch.

    Shapes: q, k, log_alpha [T, H, dk]; v [T, H, dv]; beta [T, H];
    initial_state [N, H, dk, dv] or None (zeros); cu_seqlens [N+1] or None
    (one sequence). Inputs may be torch tensors (fp32/bf16/fp64, any device)
    or numpy arrays; they are read exactly and widened to fp64.

    Returns (o, S_final, o_rec): o [T, H, dv] fp64 (None unless want_o);
    S_final [N, H, dk, dv] fp64; o_rec [len(rec_pos), len(heads), dv] or None.
    Entries of heads outside ``heads`` are left zero.
    """
    lib = _load()
    qa, in_dt = _as_host_buffer(q)
    ka, in_dt2 = _as_host_buffer(k)
    va, in_dt3 = _as_host_buffer(v)
    la, gate_dt = _as_host_buffer(log_alpha)
    ba, gate_dt2 = _as_host_buffer(beta)
    if not (in_dt == in_dt2 == in_dt3) or gate_dt != gate_dt2:
        raise TypeError("q, k, v must share a dtype; log_alpha and beta must share a dtype")
    T, H, dk = qa.shape
    dv = va.shape[2]
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        try:
            import torch
            if isinstance(cu_seqlens, torch.Tensor):
                cu_seqlens = cu_seqlens.detach().cpu().numpy()
        except ImportError:  # pragma: no cover
            pass
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    N = len(cu) - 1
    s0 = None
    if initial_state is not None:
        s0a, _ = _as_host_buffer(initial_state)
        s0 = np.ascontiguousarray(s0a, dtype=np.float64)
    S_final = np.zeros((N, H, dk, dv), dtype=np.float64)
    o = np.zeros((T, H, dv), dtype=np.float64) if want_o else None
    hs = None
    nh = H
    if heads is not None:
        hs = np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
        nh = len(hs)
    rp = None
    o_rec = None
    n_rec = 0
    if rec_pos is not None:
        rp = np.ascontiguousarray(np.asarray(rec_pos, dtype=np.int64))
        if np.any(np.diff(rp) < 0):
            raise ValueError("rec_pos must be sorted")
        n_rec = len(rp)
        o_rec = np.zeros((n_rec, nh, dv), dtype=np.float64)
    rc = lib.kda_oracle_forward(T, H, dk, dv, _ptr(qa), _ptr(ka), _ptr(va), _ptr(la), _ptr(ba),
                                in_dt, gate_dt, N, _ptr(cu), _ptr(s0), _ptr(S_final), _ptr(o),
                                _ptr(hs), nh, _ptr(rp), n_rec, _ptr(o_rec), col_blocks, threads)
    if rc != 0:
        raise ValueError(f"kda_oracle_forward failed with code {rc}")
    return o, S_final, o_rec


def decode_step(q, k, v, log_alpha, beta, state, *, heads=None, threads: int = 0):
    """One recurrent token per sequence: q, k, log_alpha [N, H, dk], v [N, H, dv],
    beta [N, H], state [N, H, dk, dv]. Returns (o [N, H, dv], new_state), fp64.
    It is the recurrence applied to N sequences of length one."""
    qa, _ = _as_host_buffer(q)
    N = qa.shape[0]
    cu = np.arange(N + 1, dtype=np.int64)
    o, S, _ = recurrence(q, k, v, log_alpha, beta, state, cu, heads=heads, threads=threads)
    return o, S


def _cu_array(cu_seqlens, T):
    if cu_seqlens is None:
        return np.array([0, T], dtype=np.int64)
    try:
        import torch
        if isinstance(cu_seqlens, torch.Tensor):
            cu_seqlens = cu_seqlens.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))


def dplr_recurrence(q, k, v, a, b, log_alpha, initial_state=None, cu_seqlens=None, *,
                    heads: Optional[Sequence[int]] = None, want_o: bool = True,
                    col_blocks: int = 1, threads: int = 0):
    """Token-by-token fp64 recurrence of the general DPLR transition
    S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t
    (see ``kda_oracle.c``). Shapes: q, k, a, b, log_alpha [T, H, dk];
    v [T, H, dv]; initial_state [N, H, dk, dv] or None; cu_seqlens [N+1] or
    None. q, k, v, a, b share one dtype. Returns (o or None, S_final), fp64."""
    lib = _load()
    bufs = [_as_host_buffer(x) for x in (q, k, v, a, b)]
    if len({d for _, d in bufs}) != 1:
        raise TypeError("q, k, v, a, b must share a dtype")
    (qa, in_dt), (ka, _), (va, _), (aa, _), (ba, _) = bufs
    la, gate_dt = _as_host_buffer(log_alpha)
    T, H, dk = qa.shape
    dv = va.shape[2]
    cu = _cu_array(cu_seqlens, T)
    N = len(cu) - 1
    s0 = None
    if initial_state is not None:
        s0a, _ = _as_host_buffer(initial_state)
        s0 = np.ascontiguousarray(s0a, dtype=np.float64)
    S_final = np.zeros((N, H, dk, dv), dtype=np.float64)
    o = np.zeros((T, H, dv), dtype=np.float64) if want_o else None
    hs, nh = None, H
    if heads is not None:
        hs = np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
        nh = len(hs)
    rc = lib.kda_oracle_dplr_forward(T, H, dk, dv, _ptr(qa), _ptr(ka), _ptr(va), _ptr(aa), _ptr(ba),
                                     _ptr(la), in_dt, gate_dt, N, _ptr(cu), _ptr(s0), _ptr(S_final),
                                     _ptr(o), _ptr(hs), nh, col_blocks, threads)
    if rc != 0:
        raise ValueError(f"kda_oracle_dplr_forward failed with code {rc}")
    return o, S_final
