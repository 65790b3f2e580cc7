"""The benchmark's machine probes (libkda_probe.so): the streaming copy moves
every byte (16-byte aligned sizes, ragged against the grid), and the MFMA loop
runs and leaves finite sums. They measure the GPU's achievable rates; nothing
of the operator runs here."""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gated_delta_rule_41_amd",
                   "libkda_probe.so")


def lib():
    p = ctypes.CDLL(LIB)
    p.kda_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
    p.kda_probe_copy.restype = ctypes.c_int32
    p.kda_probe_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    p.kda_probe_mfma_bf16.restype = ctypes.c_int32
    return p


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 3 << 20])
def test_copy_probe_copies(nbytes):
    p = lib()
    g = torch.Generator(device=DEV).manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV, generator=g)
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    assert p.kda_probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes,
                            ctypes.c_void_p(st)) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src) and not dst[nbytes:].any()
    assert p.kda_probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), 15,
                            ctypes.c_void_p(st)) == 1


def test_mfma_probe_runs():
    p = lib()
    sink = torch.full((8 * 4,), float("nan"), dtype=torch.float32, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    assert p.kda_probe_mfma_bf16(8, 10, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(st)) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
    assert p.kda_probe_mfma_bf16(0, 10, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(st)) == 1
