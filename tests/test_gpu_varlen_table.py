"""Packed batches of many sequences, and the sequence table built from
cu_seqlens on the device (read back from the end of the workspace).

* 4,096 sequences of 0-200 tokens (a serving-sized batch of short prompts,
  empty ones included) against the oracle, every token and every final state.
* The table's sanitising rule, stated here on the host: each sequence's start
  is clamped into [0, T] and its end into [start, T]; chunk counts are summed
  in order and cut at the workspace's chunk capacity floor((T + 63 N) / 64).
  Malformed offsets (decreasing, negative, past T, not starting at 0) then
  give defined, in-bounds work: each sequence runs over its sanitised tokens,
  and its final state is checked against the oracle on exactly those tokens
  (outputs of overlapping sequences share rows, so only the final states are
  compared there)."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import ws_layout
from parity import TOL_BF16, err, kda, oracle, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CH = 64


def table_rule(cu, T):
    """[N + 1][start, len, first chunk slot, chunk count] by the sanitising rule."""
    N = len(cu) - 1
    NC = (T + (CH - 1) * N) // CH
    rows, carry = [], 0
    for i in range(N):
        s = min(max(int(cu[i]), 0), T)
        e = min(max(int(cu[i + 1]), s), T)
        ln = e - s
        nch = (ln + CH - 1) // CH
        room = NC - carry
        nc = 0 if room <= 0 else min(nch, room)
        rows.append((s, min(ln, nc * CH), min(carry, NC), nc))
        carry += nch
    rows.append((T, 0, min(carry, NC), 0))
    return np.array(rows, dtype=np.int32)


def run_with_workspace(case, cu_list):
    T, H, d = case.T_total, case.H, case.dk
    N = len(cu_list) - 1
    cu = torch.tensor(cu_list, dtype=torch.int32, device=DEV)
    ws = torch.zeros(kda.workspace_size(N, T, H, d, d, case.q.dtype), dtype=torch.uint8, device=DEV)
    s0 = 0.02 * torch.randn(N, H, d, d, device=DEV, generator=torch.Generator(device=DEV).manual_seed(11))
    o, S = kda.chunk_fwd(case.q, case.k, case.v, case.log_alpha, case.beta, s0, cu, workspace=ws)
    torch.cuda.synchronize()
    tab = ws_layout.seq_table(ws, N, T, H, d, case.q.dtype == torch.float32)
    return o, S, s0, tab


def test_varlen_4096_short_sequences():
    g = np.random.default_rng(4096)
    lens = [int(x) for x in g.integers(0, 201, 4096)]
    case = ki.make_prefill("varlen-16", DEV, lengths=lens, H=2, s0_std=0.02)
    T = case.T_total
    say(f"[varlen 4096] T_total={T} empty={sum(1 for x in lens if x == 0)} H={case.H}")
    cu_list = [0] + list(np.cumsum(lens))
    o, S, s0, tab = run_with_workspace(case, cu_list)
    assert np.array_equal(tab, table_rule(cu_list, T))
    o_ref, S_ref, _ = oracle.recurrence(case.q, case.k, case.v, case.log_alpha, case.beta, s0,
                                        np.array(cu_list))
    eo, es = err(o, o_ref), err(S, S_ref)
    say(f"    err(o)={eo:.3e} err(S)={es:.3e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16


MALFORMED = {
    "decreasing": [0, 300, 120, 700, 650, 1000],
    "past-the-end": [0, 400, 1500, 2000],
    "negative": [-50, 80, -10, 1000],
    "not-from-zero-short": [130, 200, 200, 610],
    "over-capacity": [0, 1000, 0, 1000, 0],  # overlapping full-length sequences exceed the chunk capacity
}


@pytest.mark.parametrize("name", list(MALFORMED))
def test_seq_table_sanitises_malformed_offsets(name):
    cu_list = MALFORMED[name]
    T = 1000
    case = ki.make_prefill("prefill-4k", DEV, lengths=[T], H=2, s0_std=0.0)
    say(f"[malformed cu_seqlens] {name}: {cu_list} T={T}")
    o, S, s0, tab = run_with_workspace(case, cu_list)
    ref = table_rule(cu_list, T)
    say(f"    table {tab.tolist()}")
    assert np.array_equal(tab, ref)
    host = [t.cpu() for t in (case.q, case.k, case.v, case.log_alpha, case.beta)]
    for n in range(len(cu_list) - 1):
        st, ln = int(ref[n, 0]), int(ref[n, 1])
        seg = [t[st:st + ln] for t in host]
        _, S_ref, _ = oracle.recurrence(*seg, s0[n:n + 1].cpu())
        e = err(S[n:n + 1], S_ref)
        assert e <= TOL_BF16, (n, e)
