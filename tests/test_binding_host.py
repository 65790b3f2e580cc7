"""Host-side checks of the Python binding (no GPU needed): every buffer's shape
is checked against the sizes the binding passes to the library (taken from q
and v), before any device pointer is formed, so a mismatched tensor is refused
instead of being read or written out of bounds."""
import pytest
import torch

import gated_delta_rule_41_amd as kda

T, H, D = 70, 2, 64


def prefill_args(**over):
    a = dict(q=torch.zeros(T, H, D, dtype=torch.bfloat16), k=torch.zeros(T, H, D, dtype=torch.bfloat16),
             v=torch.zeros(T, H, D, dtype=torch.bfloat16), log_alpha=torch.zeros(T, H, D, dtype=torch.bfloat16),
             beta=torch.zeros(T, H, dtype=torch.bfloat16))
    a.update(over)
    return a


@pytest.mark.parametrize("name,bad", [
    ("k", torch.zeros(T - 1, H, D, dtype=torch.bfloat16)),
    ("log_alpha", torch.zeros(T, H, D + 1, dtype=torch.bfloat16)),
    ("v", torch.zeros(T, H + 1, D, dtype=torch.bfloat16)),
    ("beta", torch.zeros(T, H + 1, dtype=torch.bfloat16)),
])
def test_prefill_input_shapes(name, bad):
    with pytest.raises(ValueError, match=name):
        kda.chunk_fwd(**prefill_args(**{name: bad}))


@pytest.mark.parametrize("kw,bad", [
    ("initial_state", torch.zeros(1, H, D, D + 1)),
    ("o", torch.zeros(T, H, D - 1)),
    ("final_state", torch.zeros(2, H, D, D)),
])
def test_prefill_state_and_output_shapes(kw, bad):
    a = prefill_args()
    with pytest.raises(ValueError, match=kw):
        kda.chunk_fwd(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], **{kw: bad})


def test_prefill_cu_seqlens_form():
    a = prefill_args()
    with pytest.raises(ValueError, match="cu_seqlens"):
        kda.chunk_fwd(**a, cu_seqlens=torch.zeros(3, dtype=torch.int64))
    with pytest.raises(ValueError, match="cu_seqlens"):
        kda.chunk_fwd(**a, cu_seqlens=torch.zeros(1, dtype=torch.int32))


def test_prefill_rejects_host_tensors():
    with pytest.raises(ValueError, match="must be on"):
        kda.chunk_fwd(**prefill_args())


@pytest.mark.parametrize("name,shape", [("k", (4, H, D + 1)), ("v", (4, H + 1, D)), ("beta", (4, H + 1)),
                                        ("state", (4, H, D, D - 1)), ("o", (4, H, D + 1))])
def test_decode_shapes(name, shape):
    a = dict(q=torch.zeros(4, H, D), k=torch.zeros(4, H, D), v=torch.zeros(4, H, D),
             log_alpha=torch.zeros(4, H, D), beta=torch.zeros(4, H), state=torch.zeros(4, H, D, D))
    o = None
    if name == "o":
        o = torch.zeros(*shape)
    else:
        a[name] = torch.zeros(*shape)
    with pytest.raises(ValueError, match=name):
        kda.decode_step(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["state"], o=o)


@pytest.mark.parametrize("name", ["a", "b"])
def test_dplr_low_rank_vector_shapes(name):
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)
    a = dict(q=z(T, H, D), k=z(T, H, D), v=z(T, H, D), a=z(T, H, D), b=z(T, H, D), log_alpha=z(T, H, D))
    a[name] = z(T, H, D - 1)
    with pytest.raises(ValueError, match=name):
        kda.dplr_chunk_fwd(**a)
