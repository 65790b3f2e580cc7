"""GPU chunk intermediates (gated queries/keys, WY factors, A_qk, and, on the
fp32 path, chunk-entry states and corrected values) against the CPU chunkwise
form in fp64, read back from the workspace. Pins each kernel stage separately;
on the 16-bit path the state recursion and the output are one kernel whose
h_n / V_new stay on chip, and the final states and outputs pin it."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import ws_layout
from oracle import chunkwise as cw
from parity import kda, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# per-intermediate tolerance on max|x - ref| / max|ref|: the factors span many
# orders of magnitude inside a chunk (decay), so they are normalised by their
# largest entry; fp16 storage and operand rounding allow a few 2^-11.
TOL = {torch.float32: 2e-5, torch.bfloat16: 4e-3}


def nerr(x, ref):
    # floor: factors below ~1e-20 (e.g. a whole chunk's decay e^-140) underflow
    # in fp32/fp16 and carry no weight
    m = max(float(np.max(np.abs(ref))), 1e-20)
    return float(np.max(np.abs(x - ref)) / m)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H", [1, 2])
def test_intermediates(dt, d, H):
    lens = [130, 37]
    case = ki.make_prefill("varlen-16", DEV, lengths=lens, H=H, dk=d, dv=d, dtype=dt, s0_std=0.02)
    say(f"[intermediates] dtype={dt} d={d} H={H} lengths={lens}")
    T = case.T_total
    ws = torch.zeros(kda.workspace_size(case.N, T, H, d, d, dt), dtype=torch.uint8, device=DEV)
    o, S = kda.chunk_fwd(case.q, case.k, case.v, case.log_alpha, case.beta, case.initial_state,
                         case.cu_seqlens, workspace=ws)
    torch.cuda.synchronize()
    _, _, kept = cw.chunkwise(case.q, case.k, case.v, case.log_alpha, case.beta, case.initial_state,
                              case.cu_seqlens.cpu(), keep=True)
    # chunk slots are assigned in sequence order
    slot_of = {}
    slot = 0
    cu = [0] + list(np.cumsum(lens))
    for n in range(len(lens)):
        for c0 in range(cu[n], cu[n + 1], 64):
            slot_of[(n, c0)] = slot
            slot += 1
    worst = {}
    for (n, h, c0), inter in kept:
        L = min(64, cu[n + 1] - c0)
        got = ws_layout.decode(ws, case.N, T, H, d, dt == torch.float32, True, slot_of[(n, c0)], h)
        ref = dict(Qp=inter["Qp"], Km=inter["Km"], W=inter["W"], U=inter["U"], Aqk=inter["Aqk"],
                   gam=inter["gam"])
        if dt == torch.float32:  # with 16-bit factors h_n and V_new never leave the chip
            ref.update(h=inter["h"], Vn=inter["Vn"])
        for name, r in ref.items():
            g_ = got[name]
            if name in ("Qp", "Km", "W", "U", "Vn"):
                e = nerr(g_[:L], r)
                pad = np.max(np.abs(g_[L:])) if L < 64 else 0.0
                assert pad == 0.0, f"{name}: padding rows not zero ({pad})"
            elif name == "Aqk":
                e = nerr(g_[:L, :L], r)
            else:
                e = nerr(g_, r)
            worst[name] = max(worst.get(name, 0.0), e)
    say("    " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()))
    bad = {k: v for k, v in worst.items() if v > TOL[dt]}
    assert not bad, bad
