"""Full-size workloads on the GPU, checked against the oracle on samples it can
compute one by one: a subset of heads over the whole sequence (outputs at every
token, final states), sampled sequences of the batched decode (outputs at
several steps, states after the last step), and sampled token positions of the
1M-token prefill."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
from parity import TOL_BF16, err, gpu_prefill, head_slice, kda, oracle, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


# The -slow variants draw log alpha = -softplus(N(0,1) - 2) (mean alpha about
# 0.84, e^-12 per chunk): the carried state then survives many chunks, so the
# state handoff between chunks is what the outputs and final states check.
# Each variant checks other heads and positions.
@pytest.mark.parametrize("wl,heads", [("varlen-16", [0, 13, 31]), ("varlen-16-slow", [2, 17, 30])])
def test_varlen_16_full(wl, heads):
    case = ki.make_prefill(wl, DEV)
    say(f"[{wl}] T_total={case.T_total} lengths={case.lengths} heads={heads}")
    o, S = gpu_prefill(case)
    cu = case.cu_seqlens.cpu()
    q, k, v, la = (head_slice(t, heads) for t in (case.q, case.k, case.v, case.log_alpha))
    b = case.beta[:, heads].contiguous().cpu()
    o_ref, S_ref, _ = oracle.recurrence(q, k, v, la, b, None, cu, col_blocks=8)
    eo = err(o[:, heads], o_ref)
    es = err(S[:, heads], S_ref)
    say(f"    err(o)={eo:.3e} err(S)={es:.3e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_decode_256_full():
    N, H, d, steps = 256, 32, 128, 1000
    dec = ki.make_decode(N, H, d, steps, DEV)
    seqs = [0, 97, 255]
    check_at = {1, 2, 10, 100, 1000}
    say(f"[decode-256] N={N} H={H} steps={steps} sampled sequences={seqs}")
    state = dec["state"].clone()
    S_ref = dec["state"][seqs].double().cpu().numpy()
    sel = lambda t: t[seqs].contiguous()
    worst = 0.0
    for s in range(steps):
        o = kda.decode_step(dec["q"][s], dec["k"][s], dec["v"][s], dec["log_alpha"][s], dec["beta"][s], state)
        o_ref, S_ref = oracle.decode_step(sel(dec["q"][s]), sel(dec["k"][s]), sel(dec["v"][s]),
                                          sel(dec["log_alpha"][s]), sel(dec["beta"][s]), S_ref)
        if s + 1 in check_at:
            e = err(o[seqs], o_ref)
            worst = max(worst, e)
            say(f"    step {s + 1}: err(o)={e:.3e}")
            assert e <= TOL_BF16
    es = err(state[seqs], S_ref)
    say(f"    final states: err(S)={es:.3e}")
    assert es <= TOL_BF16


@pytest.mark.parametrize("wl,heads,seed", [("long-1m", [5], 2024), ("long-1m-slow", [22], 7)])
def test_long_1m_sampled(wl, heads, seed):
    T = 1 << 20
    case = ki.make_prefill(wl, DEV)
    g = np.random.default_rng(seed)
    pos = np.unique(g.integers(0, T, 4096))
    bnd = np.array([0, 63, 64, 65535, 65536, T - 1])
    rec = np.unique(np.concatenate([pos, bnd]))
    say(f"[{wl}] T={T} H={case.H} head={heads} positions={len(rec)}")
    o, S = gpu_prefill(case)
    q, k, v, la = (head_slice(t, heads) for t in (case.q, case.k, case.v, case.log_alpha))
    b = case.beta[:, heads].contiguous().cpu()
    s0 = case.initial_state[:, heads].contiguous().cpu()
    _, S_ref, o_rec = oracle.recurrence(q, k, v, la, b, s0, None, want_o=False, rec_pos=rec, col_blocks=16)
    og = o[torch.tensor(rec, device=DEV)][:, heads].double().cpu().numpy()
    eo = err(og, o_rec)
    eb = err(og[np.isin(rec, bnd)], o_rec[np.isin(rec, bnd)])
    es = err(S[:, heads], S_ref)
    say(f"    err(o@samples)={eo:.3e} err(o@boundaries)={eb:.3e} err(S)={es:.3e}")
    assert eo <= TOL_BF16 and eb <= TOL_BF16 and es <= TOL_BF16


def test_long_1m_backward_window():
    """The backward at the 1M-token shape with the default workspace (8 pieces
    of 2,048 chunk slots). d_o is nonzero only on a window of tokens across the
    first piece boundary (token 131,072) and the final states get no gradient,
    so the state gradient after the window is exactly zero: every gradient of
    a later token must be exactly 0 (all heads), and the window's gradients
    follow from the window alone given the state at its first token. The
    oracle runs the forward recurrence up to the window for one head, then its
    autograd backward over the window."""
    from oracle import backward as bw
    T = 1 << 20
    case = ki.make_prefill("long-1m", DEV)
    H, D = case.H, case.dk
    t0, t1, head = 131072 - 150, 131072 + 106, [9]
    assert kda.bwd_workspace_size(1, T, H, D, D) < 100e9
    g = torch.Generator(device=DEV).manual_seed(13)
    d_o = torch.zeros(T, H, D, device=DEV)
    d_o[t0:t1] = torch.randn(t1 - t0, H, D, generator=g, device=DEV)
    say(f"[long-1m backward] T={T} H={H} window [{t0}, {t1}) head={head}")
    got = kda.chunk_bwd(case.q, case.k, case.v, case.log_alpha, case.beta, d_o, case.initial_state)
    torch.cuda.synchronize()
    for nm in ("dq", "dk", "dv", "dlog_alpha", "dbeta"):
        assert not got[nm][t1:].any(), nm  # exactly zero after the window
        assert torch.isfinite(got[nm]).all(), nm
    assert torch.isfinite(got["dinitial_state"]).all()
    q, k, v, la = (head_slice(t[:t1], head) for t in (case.q, case.k, case.v, case.log_alpha))
    b = case.beta[:t1, head].contiguous().cpu()
    s0 = case.initial_state[:, head].contiguous().cpu()
    _, S_t0, _ = oracle.recurrence(q[:t0], k[:t0], v[:t0], la[:t0], b[:t0], s0, None, want_o=False, col_blocks=16)
    ref = bw.recurrence_grads(q[t0:], k[t0:], v[t0:], la[t0:], b[t0:], S_t0, None,
                              head_slice(d_o[t0:t1], head))
    errs = {nm: err(got[nm][t0:t1, head], ref[nm]) for nm in ("dq", "dk", "dv", "dlog_alpha", "dbeta")}
    say("    " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()))
    assert all(v_ <= 1e-3 for v_ in errs.values()), errs
