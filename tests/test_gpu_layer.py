"""GPU parity of the layer prologue and epilogue (kda_layer_prologue,
kda_layer_epilogue, through the C ABI) against the fp64 layer oracle
(oracle/layer.py, pinned in tests/test_layer_cpu.py), and of the whole layer
between the projections: prologue -> kda_chunk_fwd -> epilogue, the prologue
fused into the prefill (kda_layer_chunk_fwd) and both fused (kda_layer_fwd).

Bars:
* fp32 outputs: max-abs error relative to the RMS within 1e-5 (fp32 arithmetic
  against fp64);
* bf16 outputs: every element within one bf16 step (the spacing at the fp64
  value, plus 1e-5 rms(ref)) of the fp64 value (the GPU rounds its fp32 result,
  which can fall on the other side of a rounding boundary than the fp64 value);
* the operator inside the layer: its own bf16 bar, 2e-2, on the heavy-tailed
  values the prologue produces (max|v| / rms(v) about 14, against 5.4 for the
  workloads' N(0,1) values);
* the whole fp32 layer against the fp64 composition: the operator's 1e-4."""
import numpy as np
import pytest
import torch

import gated_delta_rule_41_amd as kda
import kda_inputs as ki
import oracle
from oracle import layer as ly
from parity import TOL_BF16, err, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def host(t):
    return None if t is None else t.cpu()


def steps(x, ref) -> float:
    """Largest |x - ref| in units of the bf16 spacing at ref (2^(e - 7) for
    |ref| in [2^e, 2^(e+1))), plus an fp32 floor of 1e-5 rms(ref)."""
    x = x.detach().double().cpu().numpy()
    ref = np.asarray(ref, dtype=np.float64)
    e = np.floor(np.log2(np.maximum(np.abs(ref), 1e-300)))
    allow = 2.0 ** (e - 7) + 1e-5 * np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(x - ref) / allow))


def check_outputs(label, got, ref, bf16):
    if bf16:
        worst = [steps(g, r) for g, r in zip(got, ref)]
        say(f"    {label} (bf16 steps): " + " ".join(f"{w:.2f}" for w in worst))
        assert max(worst) <= 1.0, worst
    else:
        errs = [err(g, r) for g, r in zip(got, ref)]
        say(f"    {label}: " + " ".join(f"{e:.2e}" for e in errs))
        assert max(errs) <= 1e-5, errs


def prologue(c):
    return kda.layer_prologue(c.xq, c.xk, c.xv, c.xa, c.xb, c.wq, c.wk, c.wv, c.A_log, c.dt_bias, c.cu_seqlens)


def prologue_ref(c):
    return ly.layer_prologue(c.xq, c.xk, c.xv, c.xa, c.xb, c.wq, c.wk, c.wv, c.A_log, c.dt_bias,
                             host(c.cu_seqlens))


@pytest.mark.parametrize("d,dt", [(128, torch.bfloat16), (64, torch.bfloat16), (128, torch.float32),
                                  (64, torch.float32)])
def test_prologue(d, dt):
    """Packed sequences of lengths 1-3 (shorter than the filter), an empty one and
    ragged ones: the convolution starts from zero at every sequence."""
    c = ki.make_layer("varlen-16", DEV, lengths=[1, 2, 0, 3, 70, 150], H=3, d=d, dtype=dt)
    say(f"[layer] prologue d={d} {dt}")
    got = prologue(c)
    torch.cuda.synchronize()
    check_outputs("q, k, v, log_alpha, beta", got, prologue_ref(c), dt == torch.bfloat16)


@pytest.mark.parametrize("lengths", [[16, 0, 0, 17, 3, 44, 0], [0, 5, 11, 16, 1, 31]])
def test_prologue_boundaries_at_tiles(lengths):
    """The kernel walks 16-token tiles: sequences (and empty ones) that start
    exactly on a tile boundary, just after one, or span several tiles."""
    c = ki.make_layer("varlen-16", DEV, lengths=lengths, H=2, d=128, dtype=torch.float32)
    say(f"[layer] prologue boundaries {lengths}")
    got = prologue(c)
    torch.cuda.synchronize()
    check_outputs("q, k, v, log_alpha, beta", got, prologue_ref(c), False)


@pytest.mark.parametrize("d,dt", [(128, torch.bfloat16), (128, torch.float32), (64, torch.float32)])
def test_epilogue(d, dt):
    c = ki.make_layer("varlen-16", DEV, lengths=[100, 37], H=3, d=d, dtype=dt)
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    o = torch.randn(c.T_total, c.H, d, generator=g, device=DEV) * 3.0
    say(f"[layer] epilogue d={d} {dt}")
    y = kda.layer_epilogue(o, c.xg, c.rms_w)
    torch.cuda.synchronize()
    check_outputs("y", [y], [ly.layer_epilogue(o.cpu(), c.xg.cpu(), c.rms_w.cpu())], dt == torch.bfloat16)


def test_whole_layer_fp32():
    """fp32 pre-activations: prologue -> operator -> epilogue against the fp64
    composition."""
    c = ki.make_layer("prefill-4k", DEV, lengths=[300, 5, 190], H=4, dtype=torch.float32, s0_std=0.02)
    q, k, v, la, b = prologue(c)
    o, S = kda.chunk_fwd(q, k, v, la, b, c.initial_state, c.cu_seqlens)
    y = kda.layer_epilogue(o, c.xg, c.rms_w)
    torch.cuda.synchronize()
    y_ref, S_ref, _ = ly.layer(c.xq, c.xk, c.xv, c.xa, c.xb, c.xg, c.wq, c.wk, c.wv, c.A_log, c.dt_bias,
                               c.rms_w, host(c.initial_state), host(c.cu_seqlens))
    ey, es = err(y, y_ref), err(S, S_ref)
    say(f"[layer] whole fp32 layer: y {ey:.2e}  final state {es:.2e}")
    assert ey <= 1e-4 and es <= 1e-4


@pytest.mark.parametrize("shape", ["ragged", "prefill-4k"])
def test_whole_bf16_layer(shape):
    """bf16 pre-activations, each stage against fp64 on the inputs it actually
    received: the prologue element-wise, the operator on the prologue's bf16
    outputs (bar 2e-2), the epilogue element-wise on the operator's o.
    Together they pin the composed layer."""
    kw = dict(lengths=[300, 5, 190], H=4, s0_std=0.02) if shape == "ragged" else {}
    c = ki.make_layer("prefill-4k", DEV, **kw)
    say(f"[layer] whole bf16 layer, {shape}")
    q, k, v, la, b = prologue(c)
    o, S = kda.chunk_fwd(q, k, v, la, b, c.initial_state, c.cu_seqlens)
    y = kda.layer_epilogue(o, c.xg, c.rms_w)
    torch.cuda.synchronize()
    check_outputs("prologue", (q, k, v, la, b), prologue_ref(c), True)
    o_ref, S_ref, _ = oracle.recurrence(q, k, v, la, b, c.initial_state, host(c.cu_seqlens))
    vf = v.float()
    tail = float(vf.abs().max() / vf.pow(2).mean().sqrt())
    eo, es = err(o, o_ref), err(S, S_ref)
    say(f"    operator: o {eo:.2e}  final state {es:.2e}  (v tail {tail:.1f}, bar {TOL_BF16:.0e})")
    assert eo <= TOL_BF16 and es <= TOL_BF16
    check_outputs("epilogue", [y], [ly.layer_epilogue(o.cpu(), c.xg.cpu(), c.rms_w.cpu())], True)


FUSED_CASES = {
    "ragged": dict(lengths=[300, 5, 0, 190], H=4, s0_std=0.02),
    "ragged-d64": dict(lengths=[70, 1, 129], H=3, d=64),
    "strong-decay": dict(lengths=[200, 77], H=2),  # dt_bias raised below: the exact path
    "prefill-4k": {},
}


@pytest.mark.parametrize("shape", list(FUSED_CASES))
def test_fused_layer_forward(shape):
    """kda_layer_chunk_fwd (the prologue computed inside the chunk preparation)
    against kda_layer_prologue followed by kda_chunk_fwd: the fused stage rounds
    the prologue's outputs to bf16 as the prologue kernel stores them, so the two
    agree to fp32 rounding (bar 1e-6 of the RMS; bitwise equality is reported).
    The operator's output is also checked against the oracle on those inputs
    (bar 2e-2)."""
    c = ki.make_layer("prefill-4k", DEV, **FUSED_CASES[shape])
    if shape == "strong-decay":
        # log alpha about -6 per token: a 16-row block spans ~130 in log2 units,
        # beyond the fast path's guard, so every chunk takes the exact path,
        # which reads its q, k rows from the fused path's scratch
        c.dt_bias.fill_(6.0)
    say(f"[layer] fused prologue + prefill, {shape}")
    q, k, v, la, b = prologue(c)
    o_ref, S_ref = kda.chunk_fwd(q, k, v, la, b, c.initial_state, c.cu_seqlens)
    o, S = kda.layer_chunk_fwd(c.xq, c.xk, c.xv, c.xa, c.xb, c.wq, c.wk, c.wv, c.A_log, c.dt_bias,
                               c.initial_state, c.cu_seqlens)
    torch.cuda.synchronize()
    same = torch.equal(o, o_ref) and torch.equal(S, S_ref)
    eo, es = err(o, o_ref.cpu()), err(S, S_ref.cpu())
    say(f"    fused vs unfused: o {eo:.2e}  final state {es:.2e}  bitwise {same}")
    assert eo <= 1e-6 and es <= 1e-6
    if shape != "prefill-4k":  # the whole-layer test covers the oracle at that size
        oo, So, _ = oracle.recurrence(q, k, v, la, b, c.initial_state, host(c.cu_seqlens))
        e1, e2 = err(o, oo), err(S, So)
        say(f"    fused vs oracle: o {e1:.2e}  final state {e2:.2e}  (bar {TOL_BF16:.0e})")
        assert e1 <= TOL_BF16 and e2 <= TOL_BF16


def split_last(c, S):
    """Packed rows of c without each sequence's last S tokens (the prefill), and
    the S decode steps' rows [N, H, ...] each."""
    cu = [0]
    for L in c.lengths:
        cu.append(cu[-1] + L)
    pre = [i for n in range(c.N) for i in range(cu[n], cu[n + 1] - S)]
    dec = [[cu[n + 1] - S + s for n in range(c.N)] for s in range(S)]
    idx = torch.tensor(pre, dtype=torch.long, device=DEV)
    lens = [L - S for L in c.lengths]
    cu_pre = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device=DEV)
    return idx, [torch.tensor(d, dtype=torch.long, device=DEV) for d in dec], cu_pre


@pytest.mark.parametrize("d,dt", [(128, torch.bfloat16), (64, torch.float32)])
def test_conv_state(d, dt):
    """The history after each sequence: its last three rows, oldest first, zero
    where the sequence is shorter (lengths 0, 1, 2 included); an exact copy."""
    c = ki.make_layer("varlen-16", DEV, lengths=[0, 1, 2, 70, 5], H=3, d=d, dtype=dt)
    say(f"[layer] convolution history d={d} {dt}")
    cs = kda.layer_conv_state(c.xq, c.xk, c.xv, c.cu_seqlens)
    torch.cuda.synchronize()
    ref = torch.from_numpy(ly.conv_state(c.xq, c.xk, c.xv, host(c.cu_seqlens))).to(dt)
    assert torch.equal(cs.cpu(), ref)


@pytest.mark.parametrize("d,dt", [(128, torch.bfloat16), (64, torch.bfloat16), (128, torch.float32)])
def test_decode_prologue(d, dt):
    """One new token per sequence after the history: element-wise against the
    oracle (bf16: within one step; fp32: 1e-5 of the RMS), and the shifted
    history exactly."""
    c = ki.make_layer("varlen-16", DEV, lengths=[5, 1, 0, 40], H=3, d=d, dtype=dt)
    cs = kda.layer_conv_state(c.xq, c.xk, c.xv, c.cu_seqlens)
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    new = [torch.randn(c.N, c.H, d, generator=g, device=DEV).to(dt) for _ in range(4)]
    xb = torch.randn(c.N, c.H, generator=g, device=DEV).to(dt)
    cs_before = cs.cpu()
    say(f"[layer] decode prologue d={d} {dt}")
    got = kda.layer_decode_prologue(*new, xb, cs, c.wq, c.wk, c.wv, c.A_log, c.dt_bias)
    torch.cuda.synchronize()
    ref = ly.layer_decode_prologue(*new, xb, cs_before, c.wq, c.wk, c.wv, c.A_log, c.dt_bias)
    check_outputs("q, k, v, log_alpha, beta", got, ref[:5], dt == torch.bfloat16)
    assert torch.equal(cs.cpu(), torch.from_numpy(ref[5]).to(dt))


def test_layer_decode_continues_prefill():
    """A served layer (fp32): prefill of each sequence but its last four tokens
    (prologue, kda_chunk_fwd, history), then four one-token steps (decode
    prologue, kda_decode_step in place, epilogue). Every step's output and the
    final states against the fp64 layer over the whole sequences (bar 1e-4);
    lengths 0 and 1 before decoding included."""
    S = 4
    c = ki.make_layer("prefill-4k", DEV, lengths=[41, 68, 5, 4], H=2, d=64, dtype=torch.float32, s0_std=0.02)
    idx, dec, cu_pre = split_last(c, S)
    pre = [x.index_select(0, idx) for x in (c.xq, c.xk, c.xv, c.xa, c.xb)]
    q, k, v, la, b = kda.layer_prologue(*pre, c.wq, c.wk, c.wv, c.A_log, c.dt_bias, cu_pre)
    _, state = kda.chunk_fwd(q, k, v, la, b, c.initial_state, cu_pre)
    cs = kda.layer_conv_state(pre[0], pre[1], pre[2], cu_pre)
    state_f = state.clone()
    ys = []
    for s in range(S):
        step = [x.index_select(0, dec[s]) for x in (c.xq, c.xk, c.xv, c.xa, c.xb, c.xg)]
        qd, kd, vd, lad, bd = kda.layer_decode_prologue(*step[:5], cs, c.wq, c.wk, c.wv, c.A_log, c.dt_bias)
        od = kda.decode_step(qd, kd, vd, lad, bd, state)
        ys.append(kda.layer_epilogue(od, step[5], c.rms_w))
        # the same step with the epilogue fused into the decode kernel: bitwise equal
        yf = kda.layer_decode_step(qd, kd, vd, lad, bd, state_f, step[5], c.rms_w)
        assert torch.equal(yf, ys[-1]) and torch.equal(state_f, state), f"fused decode step {s}"
    torch.cuda.synchronize()
    y_ref, S_ref, _ = ly.layer(c.xq, c.xk, c.xv, c.xa, c.xb, c.xg, c.wq, c.wk, c.wv, c.A_log, c.dt_bias, c.rms_w,
                               host(c.initial_state), host(c.cu_seqlens))
    rows = np.stack([y_ref[dec[s].cpu().numpy()] for s in range(S)])
    ey, es = err(torch.stack(ys), rows), err(state, S_ref)
    say(f"[layer] decode after prefill, {S} steps: y {ey:.2e}  final state {es:.2e}")
    assert ey <= 1e-4 and es <= 1e-4


@pytest.mark.parametrize("d,dt", [(128, torch.bfloat16), (64, torch.bfloat16), (128, torch.float32),
                                  (64, torch.float32)])
def test_layer_decode_step_fused(d, dt):
    """kda_layer_decode_step (the decode step with the epilogue fused in) on 96
    sequences x 4 heads after kda_layer_decode_prologue: y and the state bitwise
    equal to kda_decode_step (fp32 o) followed by kda_layer_epilogue, over three
    steps in place; y of the first step against the fp64 decode step and layer
    epilogue (within one bf16 step, or 1e-5 for fp32)."""
    N, H = 96, 4
    c = ki.make_layer("prefill-4k", DEV, lengths=[1] * N, H=H, d=d, dtype=dt, s0_std=0.02)
    st0 = c.initial_state.clone()
    cs = torch.randn(N, H, 3, 3, d, generator=torch.Generator(device=DEV).manual_seed(11), device=DEV).to(dt)
    cs_f = cs.clone()
    s_a, s_b = st0.clone(), st0.clone()
    for step in range(3):
        # each step draws new pre-activations from the first step's by a shift of rows
        xs = [torch.roll(x, step, 0) for x in (c.xq, c.xk, c.xv, c.xa, c.xb, c.xg)]
        qd, kd, vd, lad, bd = kda.layer_decode_prologue(*xs[:5], cs, c.wq, c.wk, c.wv, c.A_log, c.dt_bias)
        q2 = kda.layer_decode_prologue(*xs[:5], cs_f, c.wq, c.wk, c.wv, c.A_log, c.dt_bias)
        assert all(torch.equal(a, b) for a, b in zip((qd, kd, vd, lad, bd), q2))
        if step == 0:
            o_ref, _ = oracle.decode_step(qd.cpu(), kd.cpu(), vd.cpu(), lad.cpu(), bd.cpu(), st0.cpu())
            y_ref = ly.layer_epilogue(np.asarray(o_ref), xs[5].cpu(), c.rms_w.cpu())
        od = kda.decode_step(qd, kd, vd, lad, bd, s_a)
        y_two = kda.layer_epilogue(od, xs[5], c.rms_w)
        y_one = kda.layer_decode_step(qd, kd, vd, lad, bd, s_b, xs[5], c.rms_w)
        assert y_one.dtype == dt and torch.equal(y_one, y_two) and torch.equal(s_a, s_b), f"step {step}"
        if step == 0:
            check_outputs("fused decode step y", [y_one], [y_ref], dt == torch.bfloat16)
    say(f"[layer] fused decode step d={d} {dt}: bitwise equal to decode step + epilogue over 3 steps")


def test_layer_decode_step_fused_decode_256():
    """The fused decode step at decode-256 size (256 sequences x 32 heads, d = 128,
    bf16; 8,192 workgroups): y and the states bitwise equal to kda_decode_step
    followed by kda_layer_epilogue, and y of sampled sequences against the fp64
    decode step and epilogue."""
    N, H, d = 256, 32, 128
    c = ki.make_layer("decode-256", DEV, lengths=[1] * N, H=H, d=d, s0_std=0.02)
    cs = torch.randn(N, H, 3, 3, d, generator=torch.Generator(device=DEV).manual_seed(4), device=DEV).to(torch.bfloat16)
    qd, kd, vd, lad, bd = kda.layer_decode_prologue(c.xq, c.xk, c.xv, c.xa, c.xb, cs, c.wq, c.wk, c.wv, c.A_log,
                                                    c.dt_bias)
    s0 = c.initial_state
    s_a, s_b = s0.clone(), s0.clone()
    y_two = kda.layer_epilogue(kda.decode_step(qd, kd, vd, lad, bd, s_a), c.xg, c.rms_w)
    y_one = kda.layer_decode_step(qd, kd, vd, lad, bd, s_b, c.xg, c.rms_w)
    torch.cuda.synchronize()
    assert torch.equal(y_one, y_two) and torch.equal(s_a, s_b)
    seqs = [0, 97, 255]
    sel = [x[seqs] for x in (qd, kd, vd, lad, bd)]
    o_ref, _ = oracle.decode_step(*sel, s0[seqs])
    y_ref = ly.layer_epilogue(np.asarray(o_ref), c.xg[seqs].cpu(), c.rms_w.cpu())
    check_outputs("fused decode step y (decode-256, sequences 0, 97, 255)", [y_one[seqs]], [y_ref], True)


def test_whole_layer_epilogue_wait_gives_up(monkeypatch):
    """The fused epilogue's bounded wait, forced from the host: with
    KDA_EPI_SPIN_MAX=0 every wait gives up at once, so every y row is NaN, the
    launch still ends, and the chain (the final states) is untouched; back at
    the default bound the next call is normal again."""
    c = ki.make_layer("prefill-4k", DEV, lengths=[300, 5, 190, 64], H=2, s0_std=0.02)  # N H = 8: fused
    N, H, d = len(c.lengths), c.xq.shape[1], c.xq.shape[2]
    assert (N * H) % 8 == 0 and N * H * (d // 16) <= torch.cuda.get_device_properties(0).multi_processor_count
    args = (c.xq, c.xk, c.xv, c.xa, c.xb, c.xg, c.wq, c.wk, c.wv, c.A_log, c.dt_bias, c.rms_w, c.initial_state,
            c.cu_seqlens)
    y_ok, S_ok = kda.layer_fwd(*args)
    monkeypatch.setenv("KDA_EPI_SPIN_MAX", "0")
    y_nan, S_nan = kda.layer_fwd(*args)
    torch.cuda.synchronize()
    monkeypatch.delenv("KDA_EPI_SPIN_MAX")
    y_again, _ = kda.layer_fwd(*args)
    torch.cuda.synchronize()
    say(f"[layer] epilogue wait forced to give up: {int(torch.isnan(y_nan.float()).sum())} of {y_nan.numel()} NaN")
    assert bool(torch.isnan(y_nan.float()).all())
    assert torch.equal(S_nan, S_ok)
    assert bool(torch.isfinite(y_ok.float()).all()) and torch.equal(y_again, y_ok)


WHOLE_CASES = {
    # N H a multiple of 8 and N H d/16 workgroups within the CU count: the fused epilogue
    "prefill-4k": {},
    "ragged": dict(lengths=[300, 5, 0, 190, 64, 1, 129, 17], H=4, s0_std=0.02),
    "d64": dict(lengths=[70, 1, 129, 200], H=2, d=64),
    "strong-decay": dict(lengths=[200, 77], H=4),  # dt_bias raised below: the exact path
    # N H = 9: the slab workgroups of a head are not all on one XCD -> the epilogue kernel
    "not-mult-8": dict(lengths=[300, 5, 190], H=3),
    # N H d/16 = 1,024 workgroups: more than fit at once -> the epilogue kernel
    "many-heads": dict(lengths=[70, 130, 0, 64, 200, 9, 33, 100], H=16, s0_std=0.02),
}


@pytest.mark.parametrize("shape", list(WHOLE_CASES))
def test_whole_layer_one_call(shape):
    """kda_layer_fwd: prologue fused into the preparation and the epilogue into
    the recursion's output stage (or the epilogue kernel after it, where the
    slab workgroups of a head cannot share an XCD or all be resident). Against
    kda_layer_chunk_fwd followed by kda_layer_epilogue: the final states are
    bitwise equal (the chain is the same); y is within one bf16 step of the fp64
    epilogue of the operator's own o (the epilogue kernel's bar), and bitwise
    equal to the epilogue kernel's where the call falls back to it. Two calls
    give the same y."""
    c = ki.make_layer("prefill-4k", DEV, **WHOLE_CASES[shape])
    if shape == "strong-decay":
        c.dt_bias.fill_(6.0)
    N, H, d = len(c.lengths), c.xq.shape[1], c.xq.shape[2]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    fused = (N * H) % 8 == 0 and N * H * (d // 16) <= cus
    say(f"[layer] whole layer in one call, {shape}: N {N} H {H} d {d}, "
        f"{'fused epilogue' if fused else 'epilogue kernel'}")
    # the workspace holds the fused epilogue's per-row partial sums, or room for o
    T = c.xq.shape[0]
    NC = (T + 63 * N) // 64
    region = NC * H * (d // 16) * 64 * 4 if fused else T * H * d * 4
    assert kda.layer_fwd_workspace_size(N, T, H, d) == (kda.layer_chunk_fwd_workspace_size(N, T, H, d) +
                                                        (region + 255) // 256 * 256)
    o, S_ref = kda.layer_chunk_fwd(c.xq, c.xk, c.xv, c.xa, c.xb, c.wq, c.wk, c.wv, c.A_log, c.dt_bias,
                                   c.initial_state, c.cu_seqlens)
    y_ref = kda.layer_epilogue(o, c.xg, c.rms_w)
    y, S = kda.layer_fwd(c.xq, c.xk, c.xv, c.xa, c.xb, c.xg, c.wq, c.wk, c.wv, c.A_log, c.dt_bias, c.rms_w,
                         c.initial_state, c.cu_seqlens)
    y2, _ = kda.layer_fwd(c.xq, c.xk, c.xv, c.xa, c.xb, c.xg, c.wq, c.wk, c.wv, c.A_log, c.dt_bias, c.rms_w,
                          c.initial_state, c.cu_seqlens)
    torch.cuda.synchronize()
    assert torch.equal(S, S_ref), "final states differ from kda_layer_chunk_fwd's"
    assert torch.equal(y, y2), "two calls differ"
    assert bool(torch.isfinite(y.float()).all()), "non-finite y"
    n_diff = int((y != y_ref).sum())
    say(f"    y elements differing from the epilogue kernel's: {n_diff} of {y.numel()}")
    check_outputs("y", [y], [ly.layer_epilogue(o.cpu(), c.xg.cpu(), c.rms_w.cpu())], True)
    if not fused:
        assert n_diff == 0
