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


@pytest.mark.parametrize("d,dt,H", [(64, torch.bfloat16, 32), (128, torch.float32, 8)])
def test_prefill_4k_shape_other_paths(d, dt, H):
    """The prefill-4k shape (T = 4096, 64 chained chunks) on the paths the
    benchmark does not time: d = 64 with bf16 inputs (fused output, four slab
    workgroups per head) and fp32 inputs (recursion and output kernels apart,
    h_n and V_new through the workspace)."""
    case = ki.make_prefill("prefill-4k", DEV, H=H, dk=d, dv=d, dtype=dt)
    check_prefill(case, tol_for(dt), label=f"prefill-4k shape d={d} {dt}")


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


def _case_from(q, k, v, la, b, s0=None, lengths=None):
    cu = None
    if lengths is not None and len(lengths) > 1:
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=DEV)
    return ki.PrefillCase("custom", q, k, v, la, b, s0, cu, list(lengths or [q.shape[0]]))


def test_prefill_then_decode_equals_longer_prefill():
    """Recovery after a prefill: prefill(T) then one decode step matches
    prefill(T+1), and both match the oracle."""
    T = 300
    case = ki.make_prefill("prefill-4k-slow", DEV, lengths=[T + 1], H=4)
    say(f"[prefill+decode] T={T}")
    o_all, S_all = kda.chunk_fwd(case.q, case.k, case.v, case.log_alpha, case.beta, case.initial_state)
    _, S_T = kda.chunk_fwd(case.q[:T], case.k[:T], case.v[:T], case.log_alpha[:T], case.beta[:T],
                           case.initial_state)
    od = kda.decode_step(case.q[T:], case.k[T:], case.v[T:], case.log_alpha[T:], case.beta[T:], S_T)
    torch.cuda.synchronize()
    o_ref, S_ref, _ = oracle.recurrence(case.q, case.k, case.v, case.log_alpha, case.beta, case.initial_state)
    e1, e2, e3 = err(od[0], o_ref[T]), err(S_T, S_ref), err(o_all[T], o_ref[T])
    say(f"    err(decode o)={e1:.3e} err(carried S)={e2:.3e} err(prefill o)={e3:.3e}")
    assert max(e1, e2, e3) <= TOL_BF16


def test_single_token_prefill_equals_decode():
    dec = ki.make_decode(6, 4, 128, 1, DEV, seed=5)
    q, k, v, la, b = (dec[n][0] for n in ("q", "k", "v", "log_alpha", "beta"))
    say("[T=1 prefill vs decode] N=6 H=4")
    lengths = [1] * 6
    case = _case_from(q, k, v, la, b, dec["state"].clone(), lengths)
    o_p, S_p = gpu_prefill(case)
    st = dec["state"].clone()
    o_d = kda.decode_step(q, k, v, la, b, st)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.decode_step(q, k, v, la, b, dec["state"])
    assert err(o_p, o_ref) <= TOL_BF16 and err(S_p, S_ref) <= TOL_BF16
    assert err(o_d, o_ref) <= TOL_BF16 and err(st, S_ref) <= TOL_BF16


def test_split_prefill_with_carry_equals_whole():
    """Chunked prefill across calls, with the state carried in place
    (final_state aliasing initial_state), equals one call and the oracle,
    including splits that are not multiples of the chunk length."""
    case = ki.make_prefill("prefill-4k-slow", DEV, lengths=[1000], H=4)
    say("[split+carry] T=1000 split at 1, 64, 500, 777")
    o_all, S_all = gpu_prefill(case)
    S = case.initial_state.clone()
    outs = []
    for a, e in [(0, 1), (1, 64), (64, 500), (500, 777), (777, 1000)]:
        oo, _ = kda.chunk_fwd(case.q[a:e].contiguous(), case.k[a:e].contiguous(), case.v[a:e].contiguous(),
                              case.log_alpha[a:e].contiguous(), case.beta[a:e].contiguous(), S,
                              final_state=S)
        outs.append(oo)
    torch.cuda.synchronize()
    o_split = torch.cat(outs)
    o_ref, S_ref, _ = oracle.recurrence(case.q, case.k, case.v, case.log_alpha, case.beta, case.initial_state)
    e = [err(o_split, o_ref), err(S, S_ref), err(o_all, o_ref), err(S_all, S_ref)]
    say("    " + " ".join(f"{x:.3e}" for x in e))
    assert max(e) <= TOL_BF16


def test_deterministic_bitwise():
    case = ki.make_prefill("varlen-16", DEV, lengths=[700, 65, 1], H=8, s0_std=0.02)
    say("[determinism]")
    o1, S1 = gpu_prefill(case)
    o2, S2 = gpu_prefill(case)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_bf16_output(dt):
    """A bf16 output is the fp32 output rounded to nearest even, bit for bit
    (the rounding of o itself is the caller's choice, not a path error). With
    bf16 inputs o is stored by the recursion's output waves, with fp32 inputs
    by the separate output kernel."""
    case = ki.make_prefill("prefill-4k", DEV, lengths=[333], H=4, dtype=dt)
    say(f"[bf16 output, {dt} inputs]")
    o16, S16 = gpu_prefill(case, out_dtype=torch.bfloat16)
    o32, S32 = gpu_prefill(case, out_dtype=torch.float32)
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(S16, S32)
    o_ref, S_ref, _ = oracle.recurrence(case.q, case.k, case.v, case.log_alpha, case.beta, case.initial_state)
    assert err(o32, o_ref) <= tol_for(dt) and err(S32, S_ref) <= tol_for(dt)


def test_decode_bf16_output():
    """The decode step's bf16 output is its fp32 output rounded to nearest even."""
    dec = ki.make_decode(8, 4, 128, 1, DEV)
    say("[decode bf16 output]")
    s_a, s_b = dec["state"].clone(), dec["state"].clone()
    args = (dec["q"][0], dec["k"][0], dec["v"][0], dec["log_alpha"][0], dec["beta"][0])
    o16 = kda.decode_step(*args, s_a, out_dtype=torch.bfloat16)
    o32 = kda.decode_step(*args, s_b, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(s_a, s_b)


@pytest.mark.parametrize("dt,seed", [(torch.bfloat16, 0), (torch.bfloat16, 1)] +
                         [(torch.float32, sd) for sd in range(8)])
def test_extreme_decay_exact_path(dt, seed):
    """Gate ranges beyond the secondary-chunk guard (every channel of head 0
    draws log alpha uniform on [-12, 0] nats per token) take the exact
    elementwise path for the gated products. With fp32 inputs the chunk's
    partial gate sums reach ~280 (log2 units) while the exponents that matter
    are differences of nearby ones; eight draws check the fp32 bar there."""
    case = ki.make_prefill("prefill-4k", DEV, lengths=[150, 64], H=2, dtype=dt, s0_std=0.02, seed=seed)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    la = case.log_alpha.float()
    la[:, 0] = -12.0 * torch.rand(la[:, 0].shape, generator=gen, device=DEV)
    case.log_alpha.copy_(la.to(dt))
    check_prefill(case, tol_for(dt), label=f"extreme decay {dt} seed {seed}")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_no_decay_and_zero_beta(dt):
    """alpha = 1 (DeltaNet) on one head, beta = 0 (gates only) on another."""
    case = ki.make_prefill("prefill-4k", DEV, lengths=[200, 129], H=3, dtype=dt, s0_std=0.02)
    case.log_alpha[:, 0] = 0
    case.beta[:, 1] = 0
    check_prefill(case, tol_for(dt), label=f"alpha=1 / beta=0 {dt}")


def test_exact_retrieval_fp32():
    """beta = 1, unit keys, q = k: the output equals v at every token."""
    case = ki.make_prefill("prefill-4k", DEV, lengths=[300], H=2, dtype=torch.float32, s0_std=0.02)
    case.beta.fill_(1.0)
    k = case.k.double()
    case.k.copy_((k / k.norm(dim=-1, keepdim=True)).float())
    case.q.copy_(case.k)
    say("[exact retrieval fp32]")
    o, S = gpu_prefill(case)
    e = err(o, case.v.double().cpu().numpy())
    say(f"    err(o - v)={e:.3e}")
    assert e <= TOL_F32


@pytest.mark.parametrize("d,dt,gdt", [(64, torch.bfloat16, torch.bfloat16), (128, torch.float32, torch.float32),
                                      (128, torch.bfloat16, torch.float32), (64, torch.float32, torch.bfloat16)])
def test_head_sizes_and_mixed_dtypes(d, dt, gdt):
    case = ki.make_prefill("varlen-16", DEV, lengths=[90, 3, 130], H=2, dk=d, dv=d, dtype=dt, s0_std=0.02)
    case.log_alpha = case.log_alpha.to(gdt)
    case.beta = case.beta.to(gdt)
    check_prefill(case, tol_for(dt), label=f"d={d} in={dt} gates={gdt}")


def test_all_empty_sequences():
    """Zero tokens: final states equal the initial states."""
    H, d = 2, 128
    e = torch.empty(0, H, d, dtype=torch.bfloat16, device=DEV)
    s0 = torch.randn(3, H, d, d, device=DEV)
    cu = torch.zeros(4, dtype=torch.int32, device=DEV)
    say("[empty]")
    o, S = kda.chunk_fwd(e, e, e, e, torch.empty(0, H, dtype=torch.bfloat16, device=DEV), s0, cu)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(S, s0)


# Value scales on the bf16 path (fp16 value operands, fp32 state): uniform
# scaling of v and the initial state by 1e-4 (fp16's normal range starts at
# 6.1e-5) and by 1e4 (entries up to ~6e3, against fp16's 65504); and mixed
# scales, where the initial state's share of o and the new values' differ by
# up to ~100x (v x 1e-2; the initial state x 1e2), and v x 1e3.
@pytest.mark.parametrize("vs,ss", [(1e-4, 1e-4), (1e4, 1e4), (1e-2, 1.0), (1e3, 1.0), (1.0, 1e2)])
def test_value_scale(vs, ss):
    case = ki.make_prefill("prefill-4k", DEV, lengths=[1000, 333], H=4, s0_std=0.02)
    case.v.copy_((case.v.float() * vs).to(case.v.dtype))
    case.initial_state.mul_(ss)
    check_prefill(case, TOL_BF16, label=f"v x {vs:g}, initial state x {ss:g}")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_scalar_gate_gated_deltanet(dt):
    """A forget gate constant across key channels (one log alpha per token and
    head) is Gated DeltaNet, the special case KDA generalises (GeekNews "Kimi
    Linear" summary, section "Da atenção linear ao Gated DeltaNet"); the oracle's
    reduction to it is pinned on the CPU. Fast (shift +2) and slow (shift -2)
    gates on different heads."""
    case = ki.make_prefill("varlen-16", DEV, lengths=[700, 1, 190], H=4, dtype=dt, s0_std=0.02)
    T = case.T_total
    z = torch.randn(T, case.H, 1, device=DEV, generator=torch.Generator(device=DEV).manual_seed(3))
    shift = torch.tensor([2.0, 2.0, -2.0, -2.0], device=DEV).view(1, -1, 1)
    la = -torch.nn.functional.softplus(z + shift)
    case.log_alpha.copy_(la.expand(T, case.H, case.dk).to(dt))
    assert bool((case.log_alpha == case.log_alpha[:, :, :1]).all())
    check_prefill(case, tol_for(dt), label=f"scalar gate (Gated DeltaNet) {dt}")
