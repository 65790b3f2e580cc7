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
