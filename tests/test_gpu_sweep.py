"""A seeded sweep of valid configurations against the oracles: the prefill
(kda_chunk_fwd), the decode step (kda_decode_step), the backward
(kda_chunk_bwd), the one-call layer (kda_layer_fwd), the layer's own kernels
(prologue, epilogue, convolution history, one-token prologue) and the
general-DPLR comparison operator (kda_dplr_chunk_fwd), each on random draws
of the sequence count and lengths (empty sequences, one token, the chunk edges
63/64/65 and 127/128/129, and lengths up to 300), the head count, the head
size, the input and gate dtypes (each bf16 or fp32, mixed too), the gate
regime (the workloads' fast decay, slow decay, or in between), the initial
state (absent or N(0, 0.02)) and the output dtype.
The draws come from fixed seeds, so every run checks the same cases; each case
prints its draw before it runs. KDA_SWEEP_SCALE=k in the environment runs k
times as many draws of each sweep.

Bars: 1e-4 with fp32 inputs and 2e-2 with bf16 inputs (max-abs error over the
oracle's RMS, for o and the final state); a bf16 o must equal the fp32 o
rounded to bf16; the backward's six gradients 1e-3; the one-call layer's
final states bitwise those of kda_layer_chunk_fwd and its y within one bf16
step of the fp64 epilogue of the operator's own o (bitwise the epilogue
kernel's where the call falls back to it); the layer's kernels within one
bf16 step (bf16) or 1e-5 of the RMS (fp32) of the fp64 layer oracle, the
histories exactly; the DPLR operator (bf16 inputs) 2e-2 against its own
recurrence."""
import os

import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from oracle import backward as bw
from oracle import layer as ly
from parity import err, kda, say, tol_for

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
EDGE = [0, 1, 2, 63, 64, 65, 127, 128, 129]
# KDA_SWEEP_SCALE multiplies every sweep's number of draws (default 1); the
# draws of a smaller scale are the first ones of a larger one.
SCALE = max(1, int(os.environ.get("KDA_SWEEP_SCALE", "1")))


def draw(seed):
    rng = np.random.default_rng([41, seed])
    N = int(rng.integers(1, 6))
    lengths = [int(rng.choice(EDGE)) if rng.random() < 0.5 else int(rng.integers(3, 301)) for _ in range(N)]
    if sum(lengths) == 0:
        lengths[0] = 65
    return dict(lengths=lengths, H=int(rng.integers(1, 5)), d=int(rng.choice([64, 128])),
                in_dt=[torch.bfloat16, torch.float32][int(rng.integers(0, 2))],
                gate_dt=[torch.bfloat16, torch.float32][int(rng.integers(0, 2))],
                shift=float(rng.choice([2.0, 0.0, -2.0])), s0=float(rng.choice([0.0, 0.02])),
                packed=bool(N > 1 or rng.random() < 0.5))


def make_case(p, seed):
    c = ki.make_prefill("prefill-4k", DEV, lengths=p["lengths"], H=p["H"], dk=p["d"], dv=p["d"], dtype=p["in_dt"],
                        gate_shift=p["shift"], s0_std=p["s0"], seed=1000 + seed, packed=p["packed"])
    # the gates in their own dtype: rounded once from the drawn values
    c.log_alpha = c.log_alpha.float().to(p["gate_dt"]).contiguous()
    c.beta = c.beta.float().to(p["gate_dt"]).contiguous()
    return c


def describe(p):
    return (f"lengths={p['lengths']} H={p['H']} d={p['d']} in={str(p['in_dt'])[6:]} gate={str(p['gate_dt'])[6:]} "
            f"shift={p['shift']} s0={p['s0']} packed={p['packed']}")


@pytest.mark.parametrize("seed", range(16 * SCALE))
def test_prefill_sweep(seed):
    p = draw(seed)
    say(f"[sweep prefill {seed}] {describe(p)}")
    c = make_case(p, seed)
    o, S = kda.chunk_fwd(c.q, c.k, c.v, c.log_alpha, c.beta, c.initial_state, c.cu_seqlens)
    o16, S16 = kda.chunk_fwd(c.q, c.k, c.v, c.log_alpha, c.beta, c.initial_state, c.cu_seqlens,
                             out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    cu = None if c.cu_seqlens is None else c.cu_seqlens.cpu()
    o_ref, S_ref, _ = oracle.recurrence(c.q, c.k, c.v, c.log_alpha, c.beta, c.initial_state, cu)
    tol = tol_for(p["in_dt"])
    eo = err(o, o_ref) if o.numel() else 0.0
    es = err(S, S_ref)
    say(f"    err(o)={eo:.3e} err(S)={es:.3e} tol={tol:.0e}")
    assert eo <= tol and es <= tol
    assert torch.equal(o16, o.to(torch.bfloat16)) and torch.equal(S16, S)


@pytest.mark.parametrize("seed", range(8 * SCALE))
def test_decode_sweep(seed):
    """Two decode steps in place, each against the oracle's step from the
    previous oracle state."""
    rng = np.random.default_rng([42, seed])
    N, H, d = int(rng.integers(1, 40)), int(rng.integers(1, 9)), int(rng.choice([64, 128]))
    in_dt = [torch.bfloat16, torch.float32][int(rng.integers(0, 2))]
    gate_dt = [torch.bfloat16, torch.float32][int(rng.integers(0, 2))]
    say(f"[sweep decode {seed}] N={N} H={H} d={d} in={in_dt} gate={gate_dt}")
    dec = ki.make_decode(N, H, d, 2, DEV, dtype=in_dt, seed=100 + seed)
    state = dec["state"].clone()
    S_ref = dec["state"].cpu().double()
    tol = tol_for(in_dt)
    for s in range(2):
        la, b = (dec[n][s].float().to(gate_dt).contiguous() for n in ("log_alpha", "beta"))
        o = kda.decode_step(dec["q"][s], dec["k"][s], dec["v"][s], la, b, state)
        torch.cuda.synchronize()
        o_ref, S_next = oracle.decode_step(dec["q"][s], dec["k"][s], dec["v"][s], la, b, S_ref)
        eo, es = err(o, o_ref), err(state, S_next)
        say(f"    step {s}: err(o)={eo:.3e} err(S)={es:.3e} tol={tol:.0e}")
        assert eo <= tol and es <= tol
        S_ref = torch.from_numpy(np.asarray(S_next))


@pytest.mark.parametrize("seed", range(6 * SCALE))
def test_backward_sweep(seed):
    p = draw(100 + seed)
    p["lengths"] = [min(x, 200) for x in p["lengths"]][:3]  # the gradient oracle's size
    if sum(p["lengths"]) == 0:
        p["lengths"][0] = 65
    p["packed"] = p["packed"] or len(p["lengths"]) > 1
    say(f"[sweep backward {seed}] {describe(p)}")
    c = make_case(p, 100 + seed)
    g = torch.Generator(device=DEV).manual_seed(seed)
    d_o = torch.randn(c.T_total, c.H, c.dv, generator=g, device=DEV)
    d_fin = torch.randn(c.N, c.H, c.dk, c.dv, generator=g, device=DEV) * 0.1
    got = kda.chunk_bwd(c.q, c.k, c.v, c.log_alpha, c.beta, d_o, c.initial_state, c.cu_seqlens, d_fin)
    torch.cuda.synchronize()
    cu = None if c.cu_seqlens is None else c.cu_seqlens.cpu()
    ref = bw.recurrence_grads(c.q, c.k, c.v, c.log_alpha, c.beta, c.initial_state, cu, d_o.cpu(), d_fin.cpu())
    errs = {nm: err(got[nm], ref[nm]) for nm in ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dinitial_state")}
    say("    " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= 1e-3}
    assert not bad, bad


def bf16_steps(x, ref) -> float:
    """Largest |x - ref| in units of the bf16 spacing at ref, plus an fp32
    floor of 1e-5 rms(ref)."""
    x = x.detach().double().cpu().numpy()
    ref = np.asarray(ref, dtype=np.float64)
    e = np.floor(np.log2(np.maximum(np.abs(ref), 1e-300)))
    allow = 2.0 ** (e - 7) + 1e-5 * np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(x - ref) / allow))


@pytest.mark.parametrize("seed", range(8 * SCALE))
def test_layer_sweep(seed):
    """kda_layer_fwd over random shapes; N H a multiple of 8 (within the CU
    count) takes the epilogue inside the recursion, any other the epilogue kernel."""
    rng = np.random.default_rng([43, seed])
    N = int(rng.integers(1, 5))
    lengths = [int(rng.choice(EDGE)) if rng.random() < 0.4 else int(rng.integers(3, 301)) for _ in range(N)]
    if sum(lengths) == 0:
        lengths[0] = 64
    H = int(rng.choice([1, 2, 3, 4, 8])) if rng.random() < 0.6 else int(8 // N if 8 % N == 0 else 8)
    d = int(rng.choice([64, 128]))
    s0 = float(rng.choice([0.0, 0.02]))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    fused = (N * H) % 8 == 0 and N * H * (d // 16) <= cus
    say(f"[sweep layer {seed}] lengths={lengths} H={H} d={d} s0={s0} "
        f"{'epilogue in the recursion' if fused else 'epilogue kernel'}")
    c = ki.make_layer("prefill-4k", DEV, lengths=lengths, H=H, d=d, s0_std=s0, seed=200 + seed)
    o, S_ref = kda.layer_chunk_fwd(c.xq, c.xk, c.xv, c.xa, c.xb, c.wq, c.wk, c.wv, c.A_log, c.dt_bias,
                                   c.initial_state, c.cu_seqlens)
    y_two = kda.layer_epilogue(o, c.xg, c.rms_w)
    y, S = kda.layer_fwd(c.xq, c.xk, c.xv, c.xa, c.xb, c.xg, c.wq, c.wk, c.wv, c.A_log, c.dt_bias, c.rms_w,
                         c.initial_state, c.cu_seqlens)
    torch.cuda.synchronize()
    assert torch.equal(S, S_ref)
    steps = bf16_steps(y, ly.layer_epilogue(o.cpu(), c.xg.cpu(), c.rms_w.cpu()))
    say(f"    y within {steps:.2f} bf16 steps of the fp64 epilogue of o")
    assert steps <= 1.0
    if not fused:
        assert torch.equal(y, y_two)


@pytest.mark.parametrize("seed", range(6 * SCALE))
def test_dplr_sweep(seed):
    """kda_dplr_chunk_fwd (bf16 inputs; gates bf16 or fp32; fp32 or bf16 o)
    against the oracle's DPLR recurrence."""
    rng = np.random.default_rng([44, seed])
    N = int(rng.integers(1, 5))
    lengths = [int(rng.choice(EDGE)) if rng.random() < 0.5 else int(rng.integers(3, 301)) for _ in range(N)]
    if sum(lengths) == 0:
        lengths[0] = 65
    H, d = int(rng.integers(1, 5)), int(rng.choice([64, 128]))
    gate_dt = [torch.bfloat16, torch.float32][int(rng.integers(0, 2))]
    out_dt = [torch.float32, torch.bfloat16][int(rng.integers(0, 2))]
    say(f"[sweep dplr {seed}] lengths={lengths} H={H} d={d} gates={gate_dt} out={out_dt}")
    c = ki.make_dplr("prefill-4k", DEV, lengths=lengths, H=H, dk=d, dv=d, seed=300 + seed, s0_std=0.02)
    c.log_alpha = c.log_alpha.float().to(gate_dt).contiguous()
    o, S = kda.dplr_chunk_fwd(c.q, c.k, c.v, c.a, c.b, c.log_alpha, c.initial_state, c.cu_seqlens)
    torch.cuda.synchronize()
    cu = None if c.cu_seqlens is None else c.cu_seqlens.cpu()
    o_ref, S_ref = oracle.dplr_recurrence(c.q, c.k, c.v, c.a, c.b, c.log_alpha, c.initial_state, cu)
    eo, es = err(o, o_ref), err(S, S_ref)
    say(f"    err(o)={eo:.3e} err(S)={es:.3e} tol=2e-02")
    assert eo <= 2e-2 and es <= 2e-2
    if out_dt == torch.bfloat16:  # the fp32 o rounded once
        o16, S16 = kda.dplr_chunk_fwd(c.q, c.k, c.v, c.a, c.b, c.log_alpha, c.initial_state, c.cu_seqlens,
                                      out_dtype=out_dt)
        assert torch.equal(o16, o.to(torch.bfloat16)) and torch.equal(S16, S)


def close_to(got, ref, bf16, label):
    if bf16:
        worst = max(bf16_steps(g, r) for g, r in zip(got, ref))
        say(f"    {label}: within {worst:.2f} bf16 steps")
        assert worst <= 1.0
    else:
        worst = max(err(g, r) for g, r in zip(got, ref))
        say(f"    {label}: {worst:.2e} of the RMS")
        assert worst <= 1e-5


@pytest.mark.parametrize("seed", range(8 * SCALE))
def test_layer_kernels_sweep(seed):
    """The layer's prologue, epilogue, convolution history and one-token
    prologue over random packed lengths (0-3 tokens, the 16-token tile edges, up
    to 300), head counts, head sizes and dtypes."""
    rng = np.random.default_rng([45, seed])
    N = int(rng.integers(1, 7))
    edges = [0, 1, 2, 3, 15, 16, 17, 63, 64, 65]
    lengths = [int(rng.choice(edges)) if rng.random() < 0.5 else int(rng.integers(4, 301)) for _ in range(N)]
    if sum(lengths) == 0:
        lengths[0] = 17
    H, d = int(rng.integers(1, 7)), int(rng.choice([64, 128]))
    dt = [torch.bfloat16, torch.float32][int(rng.integers(0, 2))]
    bf = dt == torch.bfloat16
    say(f"[sweep layer kernels {seed}] lengths={lengths} H={H} d={d} {dt}")
    c = ki.make_layer("varlen-16", DEV, lengths=lengths, H=H, d=d, dtype=dt, seed=400 + seed, packed=True)
    cu = c.cu_seqlens.cpu()
    got = kda.layer_prologue(c.xq, c.xk, c.xv, c.xa, c.xb, c.wq, c.wk, c.wv, c.A_log, c.dt_bias, c.cu_seqlens)
    torch.cuda.synchronize()
    ref = ly.layer_prologue(c.xq, c.xk, c.xv, c.xa, c.xb, c.wq, c.wk, c.wv, c.A_log, c.dt_bias, cu)
    close_to(got, ref, bf, "prologue q, k, v, log_alpha, beta")
    g = torch.Generator(device=DEV).manual_seed(seed)
    o = torch.randn(c.T_total, H, d, generator=g, device=DEV) * float(rng.choice([0.01, 1.0, 30.0]))
    y = kda.layer_epilogue(o, c.xg, c.rms_w)
    torch.cuda.synchronize()
    close_to([y], [ly.layer_epilogue(o.cpu(), c.xg.cpu(), c.rms_w.cpu())], bf, "epilogue y")
    cs = kda.layer_conv_state(c.xq, c.xk, c.xv, c.cu_seqlens)
    torch.cuda.synchronize()
    assert torch.equal(cs.cpu(), torch.from_numpy(ly.conv_state(c.xq, c.xk, c.xv, cu)).to(dt))
    new = [torch.randn(N, H, d, generator=g, device=DEV).to(dt) for _ in range(4)]
    xb = torch.randn(N, H, generator=g, device=DEV).to(dt)
    cs_before = cs.cpu()
    got = kda.layer_decode_prologue(*new, xb, cs, c.wq, c.wk, c.wv, c.A_log, c.dt_bias)
    torch.cuda.synchronize()
    ref = ly.layer_decode_prologue(*new, xb, cs_before, c.wq, c.wk, c.wv, c.A_log, c.dt_bias)
    close_to(got, ref[:5], bf, "decode prologue")
    assert torch.equal(cs.cpu(), torch.from_numpy(ref[5]).to(dt))
