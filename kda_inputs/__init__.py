"""Seeded synthetic inputs for the KDA operator (shared by tests, bench and smoke).

This module only draws random numbers and shapes them into the workloads the
operator is exercised on. It holds none of the operator's arithmetic: no
cumulative gate, no recurrence, no chunk algebra. Both the CPU oracle and the
HIP path receive the tensors produced here (the oracle after a copy to host).

Workloads (sizes follow Kimi Linear: head dimension 128 for keys and values,
contexts up to 1,048,576 tokens -- GeekNews "Kimi Linear" summary, section
"Configuração do modelo Kimi Linear"; remio.ai "Kimi Linear Acabou de Superar a
Atenção Completa em Seus Próprios Termos", section "Código Aberto Torna as
Alegações Testáveis"):

* ``tiny-fp32``     fp32, 1 sequence, H=1, T=256, dk=dv=64, zero initial state.
* ``prefill-4k``    bf16, 1 sequence, H=32, T=4096, dk=dv=128, initial state N(0, 0.02).
* ``varlen-16``     bf16, 16 sequences with lengths uniform on [512, 16384], packed,
                    zero initial states.
* ``decode-256``    bf16 decode steps, 256 sequences, H=32, d=128, states N(0, 0.02).
* ``long-1m``       bf16, 1 sequence, T=1,048,576, initial state N(0, 0.02).

Value recipe (per token and head): q, k ~ N(0,1) then L2-normalised over dk in
fp32; v ~ N(0,1); beta = sigmoid(N(0,1)); log_alpha = -softplus(N(0,1) + shift)
per channel, with shift 0 for ``tiny-fp32`` and +2 for the bf16 workloads; the
``-slow`` variants use shift -2 (mean alpha near 0.84). Everything is drawn in
fp32 and rounded once to the input dtype with round-to-nearest-even.

General-DPLR comparison inputs (``make_dplr``): the same q, k, v, log_alpha
as the named workload, plus low-rank vectors a = beta * a_hat and b = a_hat
with a_hat ~ N(0,1) L2-normalised over dk, drawn independently of k (beta is
the workload's sigmoid draw). Then Diag(alpha) - a b^T is symmetric with
eigenvalues in [-beta, 1], so the state stays bounded over any length while
a and b share nothing with the written key k.

Layer inputs (``make_layer``): the pre-activations of a KDA layer's
projections for the prologue/epilogue path, drawn N(0,1) in fp32 and rounded
to the workload's dtype: xq, xk, xv, xa [T, H, d], xb [T, H], xg [T, H, dv];
short-convolution filters N(0, 0.5) [H, d, 4] (fp32); A_log = 0 and dt_bias =
the workload's gate shift, so that the decay gate the prologue forms,
-softplus(xa + shift), has the workload's distribution; RMSNorm weights
1 + N(0, 0.1) [dv]. (N(0, s): standard deviation s.)

Random numbers come from torch generators seeded from (workload, tensor,
window); on a GPU device the draws happen on that device (Philox), so the same
seed gives the same tensors on every run of the same software stack.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import List, Optional, Sequence

import torch

WINDOW = 65536  # tokens per generation window (bounds temporary memory)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: torch.dtype
    H: int
    dk: int
    dv: int
    lengths: Optional[Sequence[int]]  # None: drawn (varlen)
    gate_shift: float
    s0_std: float  # 0 -> no initial state (zeros)
    n_seqs: int = 1
    steps: int = 0  # decode steps (decode workloads only)


WORKLOADS = {
    "tiny-fp32": Workload("tiny-fp32", torch.float32, 1, 64, 64, [256], 0.0, 0.0),
    "prefill-4k": Workload("prefill-4k", torch.bfloat16, 32, 128, 128, [4096], 2.0, 0.02),
    "varlen-16": Workload("varlen-16", torch.bfloat16, 32, 128, 128, None, 2.0, 0.0, n_seqs=16),
    "decode-256": Workload("decode-256", torch.bfloat16, 32, 128, 128, None, 2.0, 0.02,
                           n_seqs=256, steps=1000),
    "long-1m": Workload("long-1m", torch.bfloat16, 32, 128, 128, [1 << 20], 2.0, 0.02),
}
# numbered aliases in the order the workloads are usually listed
WORKLOAD_BY_INDEX = ["tiny-fp32", "prefill-4k", "varlen-16", "decode-256", "long-1m"]


def seed_of(*parts) -> int:
    """Deterministic 63-bit seed from any tuple of ints/strings."""
    h = hashlib.sha256(repr(tuple(parts)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*parts))
    return g


def varlen_lengths(n: int = 16, lo: int = 512, hi: int = 16384, seed: int = 0) -> List[int]:
    """Sequence lengths uniform on [lo, hi] inclusive, in drawn order."""
    g = _gen("cpu", "lengths", n, lo, hi, seed)
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=g)]


def _normal(shape, device, *parts) -> torch.Tensor:
    return torch.randn(shape, generator=_gen(device, *parts), device=device, dtype=torch.float32)


def _l2n(x: torch.Tensor) -> torch.Tensor:
    # per (token, head) over the last dimension, in fp32 (input recipe, not operator math)
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)


def _softplus(x: torch.Tensor) -> torch.Tensor:
    return torch.clamp_min(x, 0.0) + torch.log1p(torch.exp(-x.abs()))


@dataclasses.dataclass
class PrefillCase:
    name: str
    q: torch.Tensor          # [T_total, H, dk]
    k: torch.Tensor          # [T_total, H, dk]
    v: torch.Tensor          # [T_total, H, dv]
    log_alpha: torch.Tensor  # [T_total, H, dk]
    beta: torch.Tensor       # [T_total, H]
    initial_state: Optional[torch.Tensor]  # [N, H, dk, dv] fp32 or None
    cu_seqlens: Optional[torch.Tensor]     # [N+1] int32 or None (single sequence)
    lengths: List[int]

    @property
    def N(self) -> int:
        return len(self.lengths)

    @property
    def T_total(self) -> int:
        return int(self.q.shape[0])

    @property
    def H(self) -> int:
        return int(self.q.shape[1])

    @property
    def dk(self) -> int:
        return int(self.q.shape[2])

    @property
    def dv(self) -> int:
        return int(self.v.shape[2])


def fill_token_inputs(T: int, H: int, dk: int, dv: int, dtype, device, gate_shift: float,
                      seed_parts: tuple, out=None, t_offset: int = 0, window: int = WINDOW):
    """Draw q, k, v, log_alpha, beta for T tokens, window by window.

    Each window of ``window`` tokens has its own seeds, so any window can be
    regenerated independently. If ``out`` is given (tuple of five tensors with
    at least t_offset+T rows) the values are written in place.
    """
    if out is None:
        out = (torch.empty(T, H, dk, dtype=dtype, device=device),
               torch.empty(T, H, dk, dtype=dtype, device=device),
               torch.empty(T, H, dv, dtype=dtype, device=device),
               torch.empty(T, H, dk, dtype=dtype, device=device),
               torch.empty(T, H, dtype=dtype, device=device))
        base = 0
    else:
        base = t_offset
    q, k, v, la, b = out
    for w0 in range(0, T, window):
        n = min(window, T - w0)
        wid = w0 // window
        sl = slice(base + w0, base + w0 + n)
        q[sl] = _l2n(_normal((n, H, dk), device, *seed_parts, "q", wid)).to(dtype)
        k[sl] = _l2n(_normal((n, H, dk), device, *seed_parts, "k", wid)).to(dtype)
        v[sl] = _normal((n, H, dv), device, *seed_parts, "v", wid).to(dtype)
        la[sl] = (-_softplus(_normal((n, H, dk), device, *seed_parts, "a", wid) + gate_shift)).to(dtype)
        b[sl] = torch.sigmoid(_normal((n, H), device, *seed_parts, "b", wid)).to(dtype)
    return out


def make_prefill(workload: str = "prefill-4k", device="cpu", *, lengths: Optional[Sequence[int]] = None,
                 H: Optional[int] = None, dk: Optional[int] = None, dv: Optional[int] = None,
                 dtype: Optional[torch.dtype] = None, gate_shift: Optional[float] = None,
                 s0_std: Optional[float] = None, seed: int = 0, packed: Optional[bool] = None) -> PrefillCase:
    """Build one prefill case. Named workloads may be overridden field by field
    (smaller H, fewer tokens ...) to make test-sized variants of the same recipe.
    A ``-slow`` suffix on the workload name selects gate shift -2."""
    slow = workload.endswith("-slow")
    base = workload[:-5] if slow else workload
    wl = WORKLOADS[base]
    H = wl.H if H is None else H
    dk = wl.dk if dk is None else dk
    dv = wl.dv if dv is None else dv
    dtype = wl.dtype if dtype is None else dtype
    if gate_shift is None:
        gate_shift = -2.0 if slow else wl.gate_shift
    s0_std = wl.s0_std if s0_std is None else s0_std
    if lengths is None:
        lengths = list(wl.lengths) if wl.lengths is not None else varlen_lengths(wl.n_seqs, seed=seed)
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    parts = (base, seed, H, dk, dv, str(dtype), tuple(lengths) if len(lengths) <= 64 else len(lengths))
    q, k, v, la, b = fill_token_inputs(T, H, dk, dv, dtype, device, gate_shift, parts)
    s0 = None
    if s0_std > 0:
        s0 = _normal((len(lengths), H, dk, dv), device, *parts, "s0") * s0_std
    if packed is None:
        packed = len(lengths) > 1
    cu = None
    if packed:
        cu_list = [0]
        for L in lengths:
            cu_list.append(cu_list[-1] + L)
        cu = torch.tensor(cu_list, dtype=torch.int32, device=device)
    elif len(lengths) != 1:
        raise ValueError("more than one sequence needs cu_seqlens")
    name = workload if (lengths == list(wl.lengths or []) or wl.lengths is None) else f"{workload}:custom"
    return PrefillCase(name, q, k, v, la, b, s0, cu, lengths)


def make_decode(N: int = 256, H: int = 32, d: int = 128, steps: int = 1000, device="cpu", *,
                dtype=torch.bfloat16, gate_shift: float = 2.0, s0_std: float = 0.02, seed: int = 0):
    """Decode workload: initial states [N, H, d, d] fp32 and per-step inputs
    stacked along a leading step axis ([steps, N, H, d] etc.). Step s draws
    from its own seed stream."""
    parts = ("decode", seed, N, H, d, str(dtype))
    s0 = _normal((N, H, d, d), device, *parts, "s0") * s0_std
    q = torch.empty(steps, N, H, d, dtype=dtype, device=device)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    la = torch.empty_like(q)
    b = torch.empty(steps, N, H, dtype=dtype, device=device)
    for s in range(steps):
        fill_token_inputs(N, H, d, d, dtype, device, gate_shift, parts + ("step", s),
                          out=(q[s], k[s], v[s], la[s], b[s]))
    return dict(state=s0, q=q, k=k, v=v, log_alpha=la, beta=b)


@dataclasses.dataclass
class DplrCase(PrefillCase):
    a: Optional[torch.Tensor] = None  # [T_total, H, dk]
    b: Optional[torch.Tensor] = None  # [T_total, H, dk]


def make_dplr(workload: str = "prefill-4k", device="cpu", **kw) -> DplrCase:
    """A prefill case of the named workload (same overrides as ``make_prefill``)
    with the low-rank vectors of the general DPLR transition added."""
    base = make_prefill(workload, device, **kw)
    T, H, dk = base.T_total, base.H, base.dk
    a = torch.empty(T, H, dk, dtype=base.q.dtype, device=device)
    b = torch.empty_like(a)
    parts = ("dplr", workload, kw.get("seed", 0), H, dk, str(base.q.dtype), T)
    for w0 in range(0, T, WINDOW):
        n = min(WINDOW, T - w0)
        sl = slice(w0, w0 + n)
        ah = _l2n(_normal((n, H, dk), device, *parts, "ahat", w0 // WINDOW))
        a[sl] = (base.beta[sl].float()[..., None] * ah).to(a.dtype)
        b[sl] = ah.to(b.dtype)
    return DplrCase(**{f.name: getattr(base, f.name) for f in dataclasses.fields(PrefillCase)}, a=a, b=b)


@dataclasses.dataclass
class LayerCase:
    name: str
    xq: torch.Tensor
    xk: torch.Tensor
    xv: torch.Tensor
    xa: torch.Tensor
    xb: torch.Tensor
    xg: torch.Tensor
    wq: torch.Tensor
    wk: torch.Tensor
    wv: torch.Tensor
    A_log: torch.Tensor
    dt_bias: torch.Tensor
    rms_w: torch.Tensor
    initial_state: Optional[torch.Tensor]
    cu_seqlens: Optional[torch.Tensor]
    lengths: List[int]

    @property
    def T_total(self) -> int:
        return self.xq.shape[0]

    @property
    def H(self) -> int:
        return self.xq.shape[1]

    @property
    def N(self) -> int:
        return len(self.lengths)


def make_layer(workload: str = "prefill-4k", device="cpu", *, lengths: Optional[Sequence[int]] = None,
               H: Optional[int] = None, d: Optional[int] = None, dtype: Optional[torch.dtype] = None,
               s0_std: Optional[float] = None, seed: int = 0, packed: Optional[bool] = None) -> LayerCase:
    """Pre-activations of the named workload's shape for the layer path (see the
    module docstring); overrides as in ``make_prefill``."""
    wl = WORKLOADS[workload]
    H = wl.H if H is None else H
    d = wl.dk if d is None else d
    dtype = wl.dtype if dtype is None else dtype
    s0_std = wl.s0_std if s0_std is None else s0_std
    if lengths is None:
        lengths = list(wl.lengths) if wl.lengths is not None else varlen_lengths(wl.n_seqs, seed=seed)
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    parts = ("layer", workload, seed, H, d, str(dtype), tuple(lengths) if len(lengths) <= 64 else len(lengths))
    x = {nm: _normal((T, H, d), device, *parts, nm).to(dtype) for nm in ("xq", "xk", "xv", "xa", "xg")}
    xb = _normal((T, H), device, *parts, "xb").to(dtype)
    w = {nm: _normal((H, d, 4), device, *parts, nm) * 0.5 for nm in ("wq", "wk", "wv")}
    A_log = torch.zeros(H, dtype=torch.float32, device=device)
    dt_bias = torch.full((H, d), float(wl.gate_shift), dtype=torch.float32, device=device)
    rms_w = 1.0 + 0.1 * _normal((d,), device, *parts, "rms_w")
    s0 = _normal((len(lengths), H, d, d), device, *parts, "s0") * s0_std if s0_std > 0 else None
    if packed is None:
        packed = len(lengths) > 1
    cu = None
    if packed:
        cu_list = [0]
        for L in lengths:
            cu_list.append(cu_list[-1] + L)
        cu = torch.tensor(cu_list, dtype=torch.int32, device=device)
    elif len(lengths) != 1:
        raise ValueError("more than one sequence needs cu_seqlens")
    return LayerCase(workload, x["xq"], x["xk"], x["xv"], x["xa"], xb, x["xg"], w["wq"], w["wk"], w["wv"],
                     A_log, dt_bias, rms_w, s0, cu, lengths)
