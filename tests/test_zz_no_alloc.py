"""The allocation-free prefill entry point (kda_chunk_fwd_noalloc) on the GPU.

It runs kda_chunk_fwd's kernels on the library's static per-device workspace.
Each case calls it through the C ABI and compares it with kda_chunk_fwd on the
same inputs (bitwise: the same kernels on the same inputs) and with the CPU
oracle (max-abs error relative to the RMS: 2e-2 for bf16 inputs, 1e-4 for
fp32), on two calls in a row, the second with a smaller input, so the second
call runs on a scratch that still holds the first call's contents."""
import pytest
import torch

import kda_inputs as ki
from parity import err, kda, oracle, say, tol_for

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run_both(case):
    o_ref, S_ref = kda.chunk_fwd(case.q, case.k, case.v, case.log_alpha, case.beta, case.initial_state,
                                 case.cu_seqlens)
    o = torch.full_like(o_ref, float("nan"))
    S = torch.full_like(S_ref, float("nan"))
    kda.chunk_fwd_noalloc(case.q, case.k, case.v, case.log_alpha, case.beta, o, case.initial_state,
                          case.cu_seqlens, S)
    torch.cuda.synchronize()
    return o, S, o_ref, S_ref


def _check(case, label):
    ws = kda.workspace_size(case.N, case.T_total, case.H, case.dk, case.dv, case.q.dtype)
    say(f"[noalloc] {label}: lengths={case.lengths} H={case.H} d={case.dk} dtype={case.q.dtype} "
        f"workspace={ws} B (limit {kda.NOALLOC_WORKSPACE_BYTES})")
    assert ws <= kda.NOALLOC_WORKSPACE_BYTES
    o, S, o_a, S_a = _run_both(case)
    assert torch.equal(o, o_a) and torch.equal(S, S_a), "noalloc differs from kda_chunk_fwd"
    cu = None if case.cu_seqlens is None else case.cu_seqlens.cpu()
    o_r, S_r, _ = oracle.recurrence(case.q, case.k, case.v, case.log_alpha, case.beta, case.initial_state, cu)
    eo, es = err(o, o_r), err(S, S_r)
    say(f"    err(o)={eo:.3e} err(S)={es:.3e}")
    tol = tol_for(case.q.dtype)
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_noalloc_two_calls_second_smaller(dt):
    # the first call fills most of the scratch (bf16: 21 chunks x 32 heads of
    # 98,816 bytes = 63.3 MiB of the 64 MiB); the second is smaller and ragged
    big = [1344] if dt == torch.bfloat16 else [300, 65, 1]
    H1 = 32 if dt == torch.bfloat16 else 8
    _check(ki.make_prefill("prefill-4k", DEV, lengths=big, H=H1, dtype=dt), "first call")
    _check(ki.make_prefill("varlen-16", DEV, lengths=[100, 0, 37], H=2, dtype=dt, s0_std=0.02),
           "second call, smaller")


def test_noalloc_refuses_oversized_before_launch():
    # one chunk-head more than the scratch holds is refused with KDA_ERR_WORKSPACE
    # on the host; the outputs stay untouched
    T = 22 * 64
    case = ki.make_prefill("prefill-4k", DEV, lengths=[T], H=32)
    assert kda.workspace_size(1, T, 32, 128, 128) > kda.NOALLOC_WORKSPACE_BYTES
    say("[noalloc] oversized call")
    o = torch.full((T, 32, 128), 7.0, device=DEV)
    with pytest.raises(kda.KDAError) as ei:
        kda.chunk_fwd_noalloc(case.q, case.k, case.v, case.log_alpha, case.beta, o, case.initial_state)
    assert ei.value.status == 6
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
