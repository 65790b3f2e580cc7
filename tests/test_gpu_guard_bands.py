"""Guard bands around every buffer a call writes: o, the final states, the
workspace (prefill, backward, the backward in pieces), the decode state and its o. Each buffer is a
view into a larger allocation whose 4 KiB before and after are filled with a
byte pattern; after the call (and a synchronisation) the bands must be
unchanged, and the call's results must still match the plain call's. Cases:
ragged lengths, empty sequences, d = 64 and 128, bf16 and fp32 inputs."""
import pytest
import torch

import kda_inputs as ki
import ws_layout
from parity import kda, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BAND = 4096  # bytes before and after (keeps the 256-byte alignment of the inner view)
PATTERN = 0xA5


class Guarded:
    """A tensor of the given shape and dtype inside a byte buffer with bands."""

    def __init__(self, shape, dtype):
        self.numel = 1
        for s in shape:
            self.numel *= s
        nbytes = self.numel * torch.tensor([], dtype=dtype).element_size()
        self.raw = torch.full((BAND + nbytes + BAND,), PATTERN, dtype=torch.uint8, device=DEV)
        self.nbytes = nbytes
        self.t = self.raw[BAND:BAND + nbytes].view(dtype).view(shape)

    def intact(self):
        return bool((self.raw[:BAND] == PATTERN).all()) and bool((self.raw[BAND + self.nbytes:] == PATTERN).all())


CASES = [
    ("ragged-empty-d128-bf16", [1, 0, 63, 64, 65, 0, 200], 128, torch.bfloat16),
    ("ragged-d64-bf16", [17, 130, 0, 5], 64, torch.bfloat16),
    ("ragged-empty-d128-fp32", [0, 100, 3, 0, 64], 128, torch.float32),
    ("ragged-d64-fp32", [33, 1, 129], 64, torch.float32),
]


@pytest.mark.parametrize("name,lengths,d,dt", CASES, ids=[c[0] for c in CASES])
def test_prefill_and_backward_write_only_their_buffers(name, lengths, d, dt):
    case = ki.make_prefill("varlen-16", DEV, lengths=lengths, H=3, dk=d, dv=d, dtype=dt, s0_std=0.02)
    T, H, N = case.T_total, case.H, case.N
    say(f"[guard bands] {name}: lengths={lengths} T={T}")
    o_ref, S_ref = kda.chunk_fwd(case.q, case.k, case.v, case.log_alpha, case.beta, case.initial_state,
                                 case.cu_seqlens)
    o = Guarded((T, H, d), torch.float32)
    fs = Guarded((N, H, d, d), torch.float32)
    ws = Guarded((kda.workspace_size(N, T, H, d, d, dt),), torch.uint8)
    kda.chunk_fwd(case.q, case.k, case.v, case.log_alpha, case.beta, case.initial_state, case.cu_seqlens,
                  o=o.t, final_state=fs.t, workspace=ws.t)
    torch.cuda.synchronize()
    assert o.intact() and fs.intact() and ws.intact()
    assert torch.equal(o.t, o_ref) and torch.equal(fs.t, S_ref)

    # the backward: every gradient and its workspace
    g = torch.Generator(device=DEV).manual_seed(5)
    d_o = torch.randn(T, H, d, generator=g, device=DEV)
    d_fin = 0.1 * torch.randn(N, H, d, d, generator=g, device=DEV)
    ref = kda.chunk_bwd(case.q, case.k, case.v, case.log_alpha, case.beta, d_o, case.initial_state,
                        case.cu_seqlens, d_fin)
    outs = {"dq": Guarded((T, H, d), torch.float32), "dk": Guarded((T, H, d), torch.float32),
            "dv": Guarded((T, H, d), torch.float32), "dlog_alpha": Guarded((T, H, d), torch.float32),
            "dbeta": Guarded((T, H), torch.float32), "dinitial_state": Guarded((N, H, d, d), torch.float32)}
    bws = Guarded((kda.bwd_workspace_size(N, T, H, d, d),), torch.uint8)
    got = kda.chunk_bwd(case.q, case.k, case.v, case.log_alpha, case.beta, d_o, case.initial_state,
                        case.cu_seqlens, d_fin, workspace=bws.t, out={k_: v_.t for k_, v_ in outs.items()})
    torch.cuda.synchronize()
    assert bws.intact() and all(v_.intact() for v_ in outs.values())
    for k_ in outs:
        assert torch.equal(got[k_], ref[k_]), k_
    # in pieces of one chunk slot (a workspace with the boundary states at its end)
    pws = Guarded((ws_layout.bwd_bytes(N, T, H, d, 1),), torch.uint8)
    got = kda.chunk_bwd(case.q, case.k, case.v, case.log_alpha, case.beta, d_o, case.initial_state,
                        case.cu_seqlens, d_fin, workspace=pws.t, out={k_: v_.t for k_, v_ in outs.items()})
    torch.cuda.synchronize()
    assert pws.intact() and all(v_.intact() for v_ in outs.values())
    for k_ in outs:
        assert torch.equal(got[k_], ref[k_]), k_


@pytest.mark.parametrize("d,dt", [(128, torch.bfloat16), (64, torch.float32)])
def test_decode_writes_only_its_buffers(d, dt):
    dec = ki.make_decode(5, 3, d, 1, DEV, dtype=dt, seed=3)
    say(f"[guard bands] decode d={d} {dt}")
    st = Guarded(tuple(dec["state"].shape), torch.float32)
    st.t.copy_(dec["state"])
    o = Guarded((5, 3, d), torch.float32)
    args = (dec["q"][0], dec["k"][0], dec["v"][0], dec["log_alpha"][0], dec["beta"][0])
    ref_state = dec["state"].clone()
    o_ref = kda.decode_step(*args, ref_state)
    kda.decode_step(*args, st.t, o=o.t)
    torch.cuda.synchronize()
    assert st.intact() and o.intact()
    assert torch.equal(o.t, o_ref) and torch.equal(st.t, ref_state)
