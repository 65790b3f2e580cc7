"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Every case prints its name before touching the GPU. Tolerances: max-abs error
relative to the oracle's RMS, 1e-4 for fp32 inputs and 2e-2 for bf16 inputs
with an fp32 state, on the outputs and on the final states."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
from parity import TOL_BF16, TOL_F32, err, gpu_prefill, head_slice, kda, oracle, say, tol_for

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def check_prefill(case, tol, out_dtype=torch.float32, label=""):
    say(f"[prefill] {label or case.name}: lengths={case.lengths[:8]}{'...' if case.N > 8 else ''} "
        f"H={case.H} d={case.dk} dtype={case.q.dtype}")
    o, S = gpu_prefill(case, out_dtype)
    o_ref, S_ref, _ = oracle.recurrence(case.q, case.k, case.v, case.log_alpha, case.beta,
                                        case.initial_state,
                                        None if case.cu_seqlens is None else case.cu_seqlens.cpu())
    eo, es = err(o, o_ref), err(S, S_ref)
    say(f"    err(o)={eo:.3e} err(S)={es:.3e} tol={tol:.0e}")
    assert eo <= tol and es <= tol
    return o, S, o_ref, S_ref


def test_tiny_fp32_workload():
    case = ki.make_prefill("tiny-fp32", DEV)
    check_prefill(case, TOL_F32)


@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65, 200])
def test_bf16_lengths(T):
    case = ki.make_prefill("prefill-4k", DEV, lengths=[T], H=2)
    check_prefill(case, TOL_BF16, label=f"bf16 T={T}")


@pytest.mark.parametrize("wl", ["prefill-4k", "prefill-4k-slow"])
def test_prefill_4k_workload(wl):
    case = ki.make_prefill(wl, DEV)
    check_prefill(case, TOL_BF16)


def test_varlen_small_with_empty_sequences():
    lens = [1, 15, 16, 17, 0, 63, 64, 65, 130, 0, 4097]
    case = ki.make_prefill("varlen-16", DEV, lengths=lens, H=3, s0_std=0.02)
    check_prefill(case, TOL_BF16)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_steps(dt, d):
    N, H, steps = 8, 4, 5
    dec = ki.make_decode(N, H, d, steps, DEV, dtype=dt)
    say(f"[decode] N={N} H={H} d={d} dtype={dt} steps={steps}")
    state = dec["state"].clone()
    S_ref = dec["state"].cpu().double().numpy()
    for s in range(steps):
        o = kda.decode_step(dec["q"][s], dec["k"][s], dec["v"][s], dec["log_alpha"][s], dec["beta"][s], state)
        torch.cuda.synchronize()
        o_ref, S_ref = oracle.decode_step(dec["q"][s], dec["k"][s], dec["v"][s], dec["log_alpha"][s],
                                          dec["beta"][s], S_ref)
        eo, es = err(o, o_ref), err(state, S_ref)
        say(f"    step {s}: err(o)={eo:.3e} err(S)={es:.3e}")
        assert eo <= tol_for(dt) and es <= tol_for(dt)
