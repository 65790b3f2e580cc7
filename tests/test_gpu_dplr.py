"""GPU parity of the general-DPLR comparison path (kda_dplr_chunk_fwd, through
the C ABI) against its CPU oracle, and of its per-chunk intermediates against
the fp64 chunkwise form.

S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t is the
general diagonal-plus-low-rank transition KDA specialises (GeekNews "Kimi
Linear" summary, section "Menos computação que o DPLR geral"). Inputs are
bf16 with an fp32 state, so the bar is the bf16 one: max-abs error relative to
the oracle's RMS <= 2e-2 on the outputs and on the final states."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import ws_layout
from oracle import chunkwise as cw
from parity import TOL_BF16, err, kda, oracle, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run(case, out_dtype=torch.float32, workspace=None):
    o, S = kda.dplr_chunk_fwd(case.q, case.k, case.v, case.a, case.b, case.log_alpha, case.initial_state,
                              case.cu_seqlens, out_dtype=out_dtype, workspace=workspace)
    torch.cuda.synchronize()
    return o, S


def check(case, label, out_dtype=torch.float32, tol=TOL_BF16):
    say(f"[dplr] {label}: lengths={case.lengths[:8]}{'...' if case.N > 8 else ''} H={case.H} d={case.dk} "
        f"gates={case.log_alpha.dtype} out={out_dtype}")
    o, S = run(case, out_dtype)
    cu = None if case.cu_seqlens is None else case.cu_seqlens.cpu()
    o_ref, S_ref = oracle.dplr_recurrence(case.q, case.k, case.v, case.a, case.b, case.log_alpha,
                                          case.initial_state, cu)
    eo, es = err(o, o_ref), err(S, S_ref)
    say(f"    err(o)={eo:.3e} err(S)={es:.3e} tol={tol:.0e}")
    assert eo <= tol and es <= tol
    return o, S


@pytest.mark.parametrize("T", [1, 16, 17, 63, 64, 65, 200])
@pytest.mark.parametrize("d", [64, 128])
def test_lengths(T, d):
    case = ki.make_dplr("prefill-4k", DEV, lengths=[T], H=2, dk=d, dv=d)
    check(case, f"T={T}")


@pytest.mark.parametrize("wl", ["prefill-4k", "prefill-4k-slow"])
def test_prefill_4k_workload(wl):
    """T = 4096, H = 32, d = 128: 64 chained chunks per head, the benchmark's launch."""
    check(ki.make_dplr(wl, DEV), wl)


def test_prefill_4k_shape_d64():
    check(ki.make_dplr("prefill-4k", DEV, dk=64, dv=64), "prefill-4k shape d=64")


@pytest.mark.parametrize("gdt", [torch.float32, torch.bfloat16])
def test_varlen_empty_sequences_and_dtypes(gdt):
    """Packed sequences (some empty) with fp32 or bf16 gates; a bf16 output is
    the fp32 output rounded once (rounding o alone costs up to ~2% of its RMS,
    so it is compared with the fp32 result, not with the oracle)."""
    lens = [1, 15, 0, 64, 65, 130, 0, 300]
    case = ki.make_dplr("varlen-16", DEV, lengths=lens, H=3, s0_std=0.02)
    case.log_alpha = case.log_alpha.to(gdt)
    o32, S32 = check(case, f"varlen gates={gdt}")
    o16, S16 = run(case, out_dtype=torch.bfloat16)
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(S16, S32)


def test_extreme_decay_exact_path():
    """Gate ranges beyond the secondary-chunk guard take the exact elementwise path."""
    case = ki.make_dplr("prefill-4k", DEV, lengths=[150, 64], H=2, s0_std=0.02)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(0)
    la = case.log_alpha.float()
    la[:, 0] = -12.0 * torch.rand(la[:, 0].shape, generator=gen, device=DEV)
    case.log_alpha.copy_(la.to(torch.bfloat16))
    check(case, "extreme decay")


def test_no_decay_and_zero_low_rank():
    """alpha = 1 on one head; a = 0 (gated linear attention) on another."""
    case = ki.make_dplr("prefill-4k", DEV, lengths=[200, 129], H=3, s0_std=0.02)
    case.log_alpha[:, 0] = 0
    case.a[:, 1] = 0
    check(case, "alpha=1 / a=0")


def test_deterministic_and_in_place_carry():
    case = ki.make_dplr("prefill-4k", DEV, lengths=[333], H=4, s0_std=0.02)
    say("[dplr] determinism / in-place carry")
    o1, S1 = run(case)
    o2, S2 = run(case)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    s = case.initial_state.clone()
    o3, S3 = kda.dplr_chunk_fwd(case.q, case.k, case.v, case.a, case.b, case.log_alpha, s, None,
                                final_state=s)
    torch.cuda.synchronize()
    assert torch.equal(o3, o1) and torch.equal(s, S1)


def test_all_empty_sequences():
    H, d = 2, 128
    e = torch.empty(0, H, d, dtype=torch.bfloat16, device=DEV)
    s0 = torch.randn(3, H, d, d, device=DEV)
    cu = torch.zeros(4, dtype=torch.int32, device=DEV)
    say("[dplr] empty")
    o, S = kda.dplr_chunk_fwd(e, e, e, e, e, e, s0, cu)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(S, s0)


# per-intermediate tolerance on max|x - ref| / max|ref| (fp16 storage, fp16 /
# split-bf16 operands), as for the KDA factors
TOL_INTER = 4e-3


@pytest.mark.parametrize("d", [64, 128])
def test_intermediates(d):
    lens = [130, 37]
    H = 2
    case = ki.make_dplr("varlen-16", DEV, lengths=lens, H=H, dk=d, dv=d, s0_std=0.02)
    say(f"[dplr intermediates] d={d} lengths={lens}")
    T = case.T_total
    ws = torch.zeros(kda.dplr_workspace_size(case.N, T, H, d, d), dtype=torch.uint8, device=DEV)
    run(case, workspace=ws)
    _, _, kept = cw.dplr_chunkwise(case.q, case.k, case.v, case.a, case.b, case.log_alpha, case.initial_state,
                                   case.cu_seqlens.cpu(), keep=True)
    cu = [0] + list(np.cumsum(lens))
    slot_of, slot = {}, 0
    for n in range(len(lens)):
        for c0 in range(cu[n], cu[n + 1], 64):
            slot_of[(n, c0)] = slot
            slot += 1
    worst = {}
    for (n, h, c0), inter in kept:
        L = min(64, cu[n + 1] - c0)
        got = ws_layout.decode_dplr(ws, case.N, T, H, d, True, slot_of[(n, c0)], h)
        for name in ("Qp", "KV", "Am", "W", "U", "Aqa", "Oh", "gam"):
            r, g_ = inter[name], got[name]
            if name == "Aqa":
                g_ = g_[:L, :L]
            elif name in ("Qp", "Am", "W", "U", "Oh"):  # chunk rows: the padding rows must be zero
                pad = float(np.max(np.abs(g_[L:]))) if L < 64 else 0.0
                assert pad == 0.0, f"{name}: padding rows not zero ({pad})"
                g_ = g_[:L]
            e = float(np.max(np.abs(g_ - r)) / max(np.max(np.abs(r)), 1e-20))
            worst[name] = max(worst.get(name, 0.0), e)
    say("    " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()))
    bad = {k: v for k, v in worst.items() if v > TOL_INTER}
    assert not bad, bad
