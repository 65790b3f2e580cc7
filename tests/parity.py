"""Helpers shared by the GPU parity tests: the error metric, running the HIP
path through the Python binding, and running the oracle on the same inputs."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import gated_delta_rule_41_amd as kda  # noqa: E402

# tolerance on max|x - ref| / rms(ref): fp32 inputs, bf16 inputs with an fp32 state
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def tol_for(dtype) -> float:
    return TOL_F32 if dtype == torch.float32 else TOL_BF16


def err(x, ref) -> float:
    """max |x - ref| / sqrt(mean(ref^2)), in fp64."""
    if isinstance(x, torch.Tensor):
        x = x.detach().to("cpu", torch.float64).numpy()
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    rms = np.sqrt(np.mean(ref * ref))
    if rms == 0:
        return float(np.max(np.abs(x - ref)))
    return float(np.max(np.abs(x - ref)) / rms)


def gpu_prefill(case, out_dtype=torch.float32):
    o, S = kda.chunk_fwd(case.q, case.k, case.v, case.log_alpha, case.beta, case.initial_state,
                         case.cu_seqlens, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o, S


def oracle_prefill(case, heads=None, rec_pos=None, want_o=True, threads=0):
    cu = None if case.cu_seqlens is None else case.cu_seqlens.cpu().numpy()
    sel = lambda t: t
    if heads is not None and want_o and rec_pos is None:
        pass
    o, S, orec = oracle.recurrence(case.q, case.k, case.v, case.log_alpha, case.beta, case.initial_state, cu,
                                   heads=heads, want_o=want_o, rec_pos=rec_pos, threads=threads,
                                   col_blocks=8 if heads is not None and len(heads) < 8 else 1)
    return o, S, orec


def head_slice(t: torch.Tensor, heads):
    """Copy only the given heads of a [T, H, ...] tensor to the host (keeps the layout)."""
    idx = torch.tensor(heads, device=t.device)
    return t.index_select(1, idx).contiguous().cpu()


def say(msg: str):
    print(msg, flush=True)
