"""GPU parity of the backward (kda_chunk_bwd, through the C ABI) against the
gradient oracle: fp64 autograd through the token recurrence, itself pinned by
finite differences (tests/test_backward_cpu.py).

The backward computes in fp32 from the exactly-read inputs, so every gradient
is held to TOL_BWD = 1e-3 in max-abs error relative to the oracle's RMS (the
forward's fp32 bar is 1e-4; the backward's adjoint chains are a few times
deeper: dS runs back over every chunk, and each local adjoint sums products of
the forward's own rounded factors)."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import ws_layout
from oracle import backward as bw
from parity import err, kda, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_BWD = 1e-3
NAMES = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dinitial_state")


def upstream(case, seed=0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    d_o = torch.randn(case.T_total, case.H, case.dv, generator=g, device=DEV)
    d_fin = torch.randn(case.N, case.H, case.dk, case.dv, generator=g, device=DEV) * 0.1
    return d_o, d_fin


def check(case, label, with_final=True, tol=TOL_BWD):
    d_o, d_fin = upstream(case)
    if not with_final:
        d_fin = None
    say(f"[bwd] {label}: lengths={case.lengths[:8]} H={case.H} d={case.dk} dtype={case.q.dtype}")
    got = kda.chunk_bwd(case.q, case.k, case.v, case.log_alpha, case.beta, d_o, case.initial_state,
                        case.cu_seqlens, d_fin)
    torch.cuda.synchronize()
    cu = None if case.cu_seqlens is None else case.cu_seqlens.cpu()
    ref = bw.recurrence_grads(case.q, case.k, case.v, case.log_alpha, case.beta, case.initial_state, cu,
                              d_o.cpu(), None if d_fin is None else d_fin.cpu())
    errs = {nm: err(got[nm], ref[nm]) for nm in NAMES}
    say("    " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad


@pytest.mark.parametrize("T", [1, 17, 64, 65, 130])
def test_lengths_fp32(T):
    case = ki.make_prefill("prefill-4k", DEV, lengths=[T], H=2, dk=64, dv=64, dtype=torch.float32, s0_std=0.02)
    check(case, f"fp32 T={T}")


@pytest.mark.parametrize("d,dt", [(128, torch.float32), (128, torch.bfloat16), (64, torch.bfloat16)])
def test_varlen_with_empty_sequences(d, dt):
    case = ki.make_prefill("varlen-16", DEV, lengths=[70, 0, 150, 5], H=2, dk=d, dv=d, dtype=dt, s0_std=0.02)
    check(case, f"varlen d={d} {dt}")


def test_slow_gates_no_final_gradient():
    case = ki.make_prefill("prefill-4k-slow", DEV, lengths=[300], H=2, dtype=torch.float32, s0_std=0.02)
    check(case, "slow gates, no d_final", with_final=False)


@pytest.mark.parametrize("shift", [3.5, 6.0])
def test_strong_decay(shift):
    """Gates falling by more than 60 nats across a 16-row block take the exact
    pairwise path for the diagonal blocks (every block at shift 6, a mix of both
    paths over the chunks at shift 3.5)."""
    case = ki.make_prefill("prefill-4k", DEV, lengths=[200, 77], H=2, gate_shift=shift, s0_std=0.02)
    check(case, f"strong decay, gate shift {shift}")


def test_prefill_4k_shape_four_heads():
    """T = 4096, d = 128 (64 chained chunks backwards), bf16 inputs, 4 heads."""
    case = ki.make_prefill("prefill-4k", DEV, H=4)
    check(case, "prefill-4k shape, H=4")


def test_deterministic():
    case = ki.make_prefill("prefill-4k", DEV, lengths=[200], H=2)
    d_o, d_fin = upstream(case)
    a = kda.chunk_bwd(case.q, case.k, case.v, case.log_alpha, case.beta, d_o, case.initial_state, None, d_fin)
    b = kda.chunk_bwd(case.q, case.k, case.v, case.log_alpha, case.beta, d_o, case.initial_state, None, d_fin)
    torch.cuda.synchronize()
    for nm in NAMES:
        assert torch.equal(a[nm], b[nm]), nm


# The backward in pieces of a few chunk slots (the workspace given sets the
# piece): the forward states at the pieces' first slots, then the pieces in
# reverse. The state crosses each cut in fp32 exactly as the recursion carries
# it, so every gradient must equal the one-piece call's bit for bit. The
# lengths put cuts inside sequences, at sequence ends, next to empty sequences
# and inside sequences spanning several pieces; [1, 1, 1, 0] fills the chunk
# capacity, so its empty last sequence sits at slot offset NC (the last piece's).
PIECE_CASES = [
    ("ragged-d128-bf16", [70, 0, 150, 5, 0, 300, 1, 0], 128, torch.bfloat16, [1, 2, 3, 5]),
    ("ragged-d64-fp32", [70, 0, 150, 5, 0, 300, 1, 0], 64, torch.float32, [1, 4, 7]),
    ("full-capacity-d64-fp32", [1, 1, 1, 0], 64, torch.float32, [1, 2]),
    ("one-sequence-d128-bf16", None, 128, torch.bfloat16, [1, 2]),
]


@pytest.mark.parametrize("label,lengths,d,dt,pieces", PIECE_CASES, ids=[c[0] for c in PIECE_CASES])
def test_pieces_bitwise_equal(label, lengths, d, dt, pieces):
    case = ki.make_prefill("varlen-16", DEV, lengths=lengths or [300], H=2, dk=d, dv=d, dtype=dt, s0_std=0.02)
    cu = case.cu_seqlens if lengths is not None else None
    T, H, N = case.T_total, case.H, case.N
    d_o, d_fin = upstream(case)
    args = (case.q, case.k, case.v, case.log_alpha, case.beta, d_o, case.initial_state, cu, d_fin)
    whole = kda.chunk_bwd(*args)
    assert kda.bwd_workspace_size(N, T, H, d, d) == ws_layout.bwd_bytes(N, T, H, d, ws_layout.chunk_capacity(
        N, T, cu is not None), cu is not None)
    for pc in pieces:
        ws = torch.empty(ws_layout.bwd_bytes(N, T, H, d, pc, cu is not None), dtype=torch.uint8, device=DEV)
        say(f"[bwd pieces] {label}: T={T} N={N} piece={pc} slots, workspace {ws.numel()} B")
        got = kda.chunk_bwd(*args, workspace=ws)
        torch.cuda.synchronize()
        for nm in NAMES:
            assert torch.equal(got[nm], whole[nm]), (pc, nm)
    # in place (the initial states' gradient over d_final_state), one slot per piece
    ws = torch.empty(ws_layout.bwd_bytes(N, T, H, d, 1, cu is not None), dtype=torch.uint8, device=DEV)
    dfin = d_fin.clone()
    kda.chunk_bwd(*args[:-1], dfin, workspace=ws, out={"dinitial_state": dfin})
    torch.cuda.synchronize()
    assert torch.equal(dfin, whole["dinitial_state"])


def test_pieces_against_oracle():
    """One piece per chunk slot, checked against the gradient oracle directly."""
    case = ki.make_prefill("varlen-16", DEV, lengths=[70, 0, 150, 5], H=2, dk=64, dv=64, dtype=torch.float32,
                           s0_std=0.02)
    d_o, d_fin = upstream(case)
    T, H, N = case.T_total, case.H, case.N
    ws = torch.empty(ws_layout.bwd_bytes(N, T, H, 64, 1), dtype=torch.uint8, device=DEV)
    got = kda.chunk_bwd(case.q, case.k, case.v, case.log_alpha, case.beta, d_o, case.initial_state,
                        case.cu_seqlens, d_fin, workspace=ws)
    torch.cuda.synchronize()
    ref = bw.recurrence_grads(case.q, case.k, case.v, case.log_alpha, case.beta, case.initial_state,
                              case.cu_seqlens.cpu(), d_o.cpu(), d_fin.cpu())
    errs = {nm: err(got[nm], ref[nm]) for nm in NAMES}
    say("    " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL_BWD for v in errs.values()), errs
