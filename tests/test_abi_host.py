"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/kda.h declares, sizes the workspace as documented and
rejects bad arguments with the right status before touching the device.

Argument-validation calls use fake, never-dereferenced device addresses: every
case here fails validation, so nothing is launched."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_41_amd as kda
import ws_layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, NULL, SHAPE, UNSUP, ALIGN, ALIAS, WORKSPACE, HIP = range(8)
F32, BF16 = 0, 1


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = kda._load()
    names = declared_functions()
    assert names == ["kda_abi_version", "kda_chunk_bwd", "kda_chunk_bwd_workspace_size", "kda_chunk_fwd",
                     "kda_chunk_fwd_noalloc", "kda_chunk_fwd_timed",
                     "kda_chunk_fwd_workspace_size", "kda_decode_step", "kda_dplr_chunk_fwd",
                     "kda_dplr_chunk_fwd_workspace_size", "kda_layer_chunk_fwd", "kda_layer_chunk_fwd_workspace_size",
                     "kda_layer_conv_state", "kda_layer_decode_prologue", "kda_layer_decode_step",
                     "kda_layer_epilogue", "kda_layer_fwd",
                     "kda_layer_fwd_workspace_size", "kda_layer_prologue", "kda_status_str"]
    for nm in names:
        assert hasattr(lib, nm), nm


def test_version_and_status_strings():
    assert kda.abi_version() == 1
    for s in range(8):
        assert kda.status_str(s).startswith("KDA_")
    assert kda.status_str(99) == "KDA_ERR_UNKNOWN"


def test_workspace_size_formula():
    # per chunk-head, d = 128, 16-bit factors: Q+, K-, -W 16 KiB each, U 32 KiB (fp32),
    # A_qk 16 KiB (two fp16 planes), gamma 512 B -> 98816 B (the fused output keeps
    # h_n and V_new on chip); chunks = floor((T + 63 N) / 64)
    # plus the sequence table at the end: (N + 1) x 16 B, rounded up to 256
    assert kda.workspace_size(1, 4096, 32, 128, 128) == 64 * 32 * 98816 + 256
    assert kda.workspace_size(16, 135000, 32, 128, 128) == ((135000 + 63 * 16) // 64) * 32 * 98816 + 512
    assert kda.workspace_size(4096, 409600, 32, 128, 128) == (
        ((409600 + 63 * 4096) // 64) * 32 * 98816 + (4097 * 16 + 255) // 256 * 256)
    # fp32 factors double every array but gamma, and add h_n and V_new
    assert kda.workspace_size(1, 256, 1, 64, 64, __import__("torch").float32) == 4 * (
        4 * (64 * 64 * 4) + 64 * 64 * 4 + 64 * 4 + 64 * 64 * 4 + 64 * 64 * 4) + 256
    with pytest.raises(kda.KDAError):
        kda.workspace_size(1, 10, 1, 96, 96)
    with pytest.raises(kda.KDAError):
        kda.workspace_size(0, 10, 1, 64, 64)


class Fake:
    """Fake device addresses laid out far apart (never dereferenced)."""

    def __init__(self):
        self.base = 0x7F0000000000
        self.i = 0

    def __call__(self, off=0):
        self.i += 1
        return self.base + self.i * (1 << 36) + off


def chunk_call(**over):
    f = Fake()
    a = dict(q=f(), k=f(), v=f(), la=f(), beta=f(), s0=None, cu=None, N=1, T=256, H=2, dk=64, dv=64,
             in_dt=BF16, gate_dt=BF16, out_dt=F32, o=f(), sf=f(), ws=f(), ws_bytes=1 << 40, stream=None)
    a.update(over)
    lib = kda._load()
    P = ctypes.c_void_p
    return lib.kda_chunk_fwd(P(a["q"]), P(a["k"]), P(a["v"]), P(a["la"]), P(a["beta"]), P(a["s0"]),
                             P(a["cu"]), a["N"], a["T"], a["H"], a["dk"], a["dv"], a["in_dt"],
                             a["gate_dt"], a["out_dt"], P(a["o"]), P(a["sf"]), P(a["ws"]),
                             a["ws_bytes"], P(a["stream"]))


def test_chunk_fwd_validation():
    assert chunk_call(q=None) == NULL
    assert chunk_call(o=None) == NULL
    assert chunk_call(N=0) == SHAPE
    assert chunk_call(T=-1) == SHAPE
    assert chunk_call(T=1 << 31) == SHAPE
    assert chunk_call(N=2) == SHAPE  # several sequences need cu_seqlens
    assert chunk_call(H=(1 << 16) + 1) == SHAPE
    f0 = Fake()
    assert chunk_call(N=1 << 15, H=1 << 13, cu=f0()) == SHAPE  # N * H * 8 state-slab workgroups >= 2^31
    assert chunk_call(dk=96, dv=96) == UNSUP
    assert chunk_call(dk=64, dv=128) == UNSUP
    assert chunk_call(in_dt=5) == UNSUP
    assert chunk_call(out_dt=2) == UNSUP
    f = Fake()
    assert chunk_call(q=f(2)) == ALIGN
    assert chunk_call(cu=f(2), N=1) == ALIGN
    assert chunk_call(beta=f(1)) == ALIGN
    assert chunk_call(la=f(8)) == ALIGN
    # o overlapping q
    q = f()
    assert chunk_call(q=q, o=q + 64) == ALIAS
    # final state overlapping an input other than the initial state
    k = f()
    assert chunk_call(k=k, sf=k) == ALIAS
    # partially overlapping initial/final state
    s = f()
    assert chunk_call(s0=s, sf=s + 256) == ALIAS
    # workspace
    assert chunk_call(ws=None) == WORKSPACE
    assert chunk_call(ws=f(16)) == WORKSPACE
    need = kda.workspace_size(1, 256, 2, 64, 64)
    assert chunk_call(ws_bytes=need - 1) == WORKSPACE
    w = f()
    assert chunk_call(ws=w, q=w + need // 2) == ALIAS


def decode_call(**over):
    f = Fake()
    a = dict(q=f(), k=f(), v=f(), la=f(), beta=f(), state=f(), N=4, H=2, dk=128, dv=128,
             in_dt=BF16, gate_dt=BF16, out_dt=F32, o=f(), stream=None)
    a.update(over)
    P = ctypes.c_void_p
    return kda._load().kda_decode_step(P(a["q"]), P(a["k"]), P(a["v"]), P(a["la"]), P(a["beta"]),
                                       P(a["state"]), a["N"], a["H"], a["dk"], a["dv"], a["in_dt"],
                                       a["gate_dt"], a["out_dt"], P(a["o"]), P(a["stream"]))


def test_decode_validation():
    assert decode_call(state=None) == NULL
    assert decode_call(N=0) == SHAPE
    assert decode_call(dk=32, dv=32) == UNSUP
    f = Fake()
    assert decode_call(state=f(8)) == ALIGN
    s = f()
    assert decode_call(state=s, o=s + 1024) == ALIAS
    v = f()
    assert decode_call(v=v, state=v) == ALIAS


def test_dplr_workspace_size_formula():
    # per chunk-head, d = 128: Q+, A-^T, -W', -U', A_qk V 16 KiB each (fp16),
    # K-^T V 32 KiB, A_qa 8 KiB, gamma 512 B -> 123392 B
    # (+ the sequence table, (N + 1) x 16 B rounded up to 256)
    assert kda.dplr_workspace_size(1, 4096, 32, 128, 128) == 64 * 32 * 123392 + 256
    assert kda.dplr_workspace_size(3, 100, 2, 64, 64) == ((100 + 63 * 3) // 64) * 2 * (6 * 8192 + 8192 + 256) + 256
    with pytest.raises(kda.KDAError):
        kda.dplr_workspace_size(1, 10, 1, 96, 96)
    out = ctypes.c_size_t(0)
    assert kda._load().kda_dplr_chunk_fwd_workspace_size(1, 10, 1, 64, 64, F32, ctypes.byref(out)) == UNSUP


def dplr_call(**over):
    f = Fake()
    a = dict(q=f(), k=f(), v=f(), a=f(), b=f(), la=f(), s0=None, cu=None, N=1, T=256, H=2, dk=64, dv=64,
             in_dt=BF16, gate_dt=BF16, out_dt=F32, o=f(), sf=f(), ws=f(), ws_bytes=1 << 40, stream=None)
    a.update(over)
    P = ctypes.c_void_p
    return kda._load().kda_dplr_chunk_fwd(P(a["q"]), P(a["k"]), P(a["v"]), P(a["a"]), P(a["b"]), P(a["la"]),
                                          P(a["s0"]), P(a["cu"]), a["N"], a["T"], a["H"], a["dk"], a["dv"],
                                          a["in_dt"], a["gate_dt"], a["out_dt"], P(a["o"]), P(a["sf"]),
                                          P(a["ws"]), a["ws_bytes"], P(a["stream"]))


def test_dplr_validation():
    assert dplr_call(a=None) == NULL
    assert dplr_call(b=None) == NULL
    assert dplr_call(N=2) == SHAPE
    assert dplr_call(T=1 << 31) == SHAPE
    assert dplr_call(in_dt=F32) == UNSUP  # 16-bit factors only
    assert dplr_call(dk=64, dv=128) == UNSUP
    f = Fake()
    assert dplr_call(b=f(8)) == ALIGN
    a_ = f()
    assert dplr_call(a=a_, o=a_ + 128) == ALIAS
    b_ = f()
    assert dplr_call(b=b_, sf=b_) == ALIAS
    need = kda.dplr_workspace_size(1, 256, 2, 64, 64)
    assert dplr_call(ws_bytes=need - 1) == WORKSPACE
    w = f()
    assert dplr_call(ws=w, b=w + need // 2) == ALIAS


def test_bwd_workspace_size_formula():
    # per chunk-head, d = 128: the fp32 forward recompute (Q+, K-, -W, U, V_new
    # 32 KiB each, A_qk 16 KiB, gamma 512 B, h_n 64 KiB), the state-gradient
    # chain's U, states and V_new (32 + 64 + 32 KiB), the added term Q+^T dO
    # whose 64 KiB the local kernel's scratch (dQ+, dK-) reuses, the gated key
    # products 16 KiB -> 459264 B
    fwd = 5 * 32768 + 16384 + 512 + 65536
    assert ws_layout.bwd_chunk_head_bytes(128) == fwd + 131072 + 65536 + 16384 == 459264
    fwd64 = 5 * 16384 + 16384 + 256 + 16384
    assert ws_layout.bwd_chunk_head_bytes(64) == fwd64 + 3 * 16384 + 32768 + 16384 == 213248
    # (+ the sequence table, (N + 1) x 16 B rounded up to 256)
    assert kda.bwd_workspace_size(1, 4096, 32, 128, 128) == 64 * 32 * 459264 + 256
    assert kda.bwd_workspace_size(2, 100, 1, 64, 64) == ((100 + 63 * 2) // 64) * 213248 + 256
    with pytest.raises(kda.KDAError):
        kda.bwd_workspace_size(1, 10, 1, 64, 128)


def test_bwd_workspace_pieces():
    """Beyond KDA_BWD_PIECE_CHUNK_HEADS chunk-heads the size query plans pieces
    of floor(65536 / H) slots plus one [H, d, d] state per piece: the 1M-token
    sequence at H = 32, d = 128 takes 8 pieces of 2048 slots, about 30.1 GB."""
    T = 1 << 20
    got = kda.bwd_workspace_size(1, T, 32, 128, 128)
    assert got == ws_layout.bwd_bytes(1, T, 32, 128, 2048) == 2048 * 32 * 459264 + 8 * 32 * 65536 + 256
    assert got < 100e9
    # exactly at the bound: one piece; one slot more: pieces
    assert kda.bwd_workspace_size(1, 2048 * 64, 32, 128, 128) == 2048 * 32 * 459264 + 256
    assert kda.bwd_workspace_size(1, 2048 * 64 + 1, 32, 128, 128) == ws_layout.bwd_bytes(1, 2048 * 64 + 1, 32,
                                                                                         128, 2048)
    # as many heads as the bound: one slot per piece
    assert kda.bwd_workspace_size(1, 128, 65536, 64, 64) == ws_layout.bwd_bytes(1, 128, 65536, 64, 1)


def test_bwd_smallest_workspace():
    """Any workspace down to one slot per piece passes validation (here the
    call then fails at its first launch, with no GPU); one byte less is
    KDA_ERR_WORKSPACE."""
    for N, T, cu in ((1, 256, None), (3, 200, 0x100000000000 - 4096)):
        least = ws_layout.bwd_bytes(N, T, 2, 64, 1, have_cu=cu is not None)
        assert bwd_call(N=N, T=T, cu=cu, ws_bytes=least - 1) == WORKSPACE
        assert bwd_call(N=N, T=T, cu=cu, ws_bytes=least) == HIP
        for pc in (2, 3):
            assert bwd_call(N=N, T=T, cu=cu, ws_bytes=ws_layout.bwd_bytes(N, T, 2, 64, pc,
                                                                            have_cu=cu is not None)) == HIP


def bwd_call(**over):
    f = Fake()
    a = dict(q=f(), k=f(), v=f(), la=f(), beta=f(), s0=None, cu=None, N=1, T=256, H=2, dk=64, dv=64,
             in_dt=BF16, gate_dt=BF16, do=f(), dfin=None, dq=f(), dk_=f(), dv_=f(), dla=f(), db=f(), ds0=f(),
             ws=f(), ws_bytes=1 << 40, stream=None)
    a.update(over)
    P = ctypes.c_void_p
    return kda._load().kda_chunk_bwd(P(a["q"]), P(a["k"]), P(a["v"]), P(a["la"]), P(a["beta"]), P(a["s0"]),
                                     P(a["cu"]), a["N"], a["T"], a["H"], a["dk"], a["dv"], a["in_dt"],
                                     a["gate_dt"], P(a["do"]), P(a["dfin"]), P(a["dq"]), P(a["dk_"]),
                                     P(a["dv_"]), P(a["dla"]), P(a["db"]), P(a["ds0"]), P(a["ws"]),
                                     a["ws_bytes"], P(a["stream"]))


def test_bwd_validation():
    assert bwd_call(do=None) == NULL
    assert bwd_call(db=None) == NULL
    assert bwd_call(N=2) == SHAPE
    assert bwd_call(T=-1) == SHAPE
    assert bwd_call(dk=64, dv=128) == UNSUP
    assert bwd_call(gate_dt=7) == UNSUP
    f = Fake()
    assert bwd_call(dla=f(4)) == ALIGN
    assert bwd_call(db=f(2)) == ALIGN
    q = f()
    assert bwd_call(q=q, dq=q + 64) == ALIAS
    dq = f()
    assert bwd_call(dq=dq, dk_=dq + 1024) == ALIAS
    d = 0x100000000000  # below every address bwd_call makes up
    assert bwd_call(dfin=d, ds0=d) != ALIAS  # in place: the initial states' gradient replaces d_final
    assert bwd_call(dfin=d, ds0=d + 256) == ALIAS
    assert bwd_call(ws=f(64)) == WORKSPACE
    need = kda.bwd_workspace_size(1, 256, 2, 64, 64)
    assert bwd_call(ws_bytes=need - 1) == HIP  # smaller pieces (then no GPU to launch on)
    assert bwd_call(ws_bytes=ws_layout.bwd_bytes(1, 256, 2, 64, 1) - 1) == WORKSPACE
    w = f()
    assert bwd_call(ws=w, do=w + need // 2) == ALIAS


def prologue_call(**over):
    f = Fake()
    a = dict(xq=f(), xk=f(), xv=f(), xa=f(), xb=f(), wq=f(), wk=f(), wv=f(), A_log=f(), dtb=f(), cu=None, N=1,
             T=100, H=2, d=64, dt=BF16, q=f(), k=f(), v=f(), la=f(), beta=f(), stream=None)
    a.update(over)
    P = ctypes.c_void_p
    return kda._load().kda_layer_prologue(*(P(a[x]) for x in ("xq", "xk", "xv", "xa", "xb", "wq", "wk", "wv",
                                                              "A_log", "dtb", "cu")),
                                          a["N"], a["T"], a["H"], a["d"], a["dt"],
                                          *(P(a[x]) for x in ("q", "k", "v", "la", "beta", "stream")))


def epilogue_call(**over):
    f = Fake()
    a = dict(o=f(), g=f(), w=f(), T=100, H=2, dv=128, dt=BF16, y=f(), stream=None)
    a.update(over)
    P = ctypes.c_void_p
    return kda._load().kda_layer_epilogue(P(a["o"]), P(a["g"]), P(a["w"]), a["T"], a["H"], a["dv"], a["dt"],
                                          P(a["y"]), P(a["stream"]))


def test_layer_validation():
    assert prologue_call(xq=None) == NULL
    assert prologue_call(beta=None) == NULL
    assert prologue_call(N=2) == SHAPE
    assert prologue_call(T=1 << 31) == SHAPE
    assert prologue_call(T=1 << 30, H=4) == SHAPE  # T * H >= 2^31
    assert prologue_call(d=96) == UNSUP
    assert prologue_call(dt=3) == UNSUP
    f = Fake()
    assert prologue_call(wq=f(2)) == ALIGN
    assert prologue_call(q=f(1)) == ALIGN
    assert prologue_call(xk=f(2)) == ALIGN  # bf16 channel pairs move as 4 bytes
    assert prologue_call(T=0, xb=f(2), beta=f(2)) == OK  # [T, H] tensors: one element (no launch at T = 0)
    x = f()
    assert prologue_call(xq=x, q=x + 64) == ALIAS
    y = f()
    assert prologue_call(q=y, k=y + 128) == ALIAS
    assert prologue_call(T=0, xq=None, q=None) == OK  # nothing to do
    assert epilogue_call(o=None) == NULL
    assert epilogue_call(dv=96) == UNSUP
    assert epilogue_call(T=-1) == SHAPE
    assert epilogue_call(y=f(1)) == ALIGN
    assert epilogue_call(o=f(4)) == ALIGN  # fp32 channel pairs move as 8 bytes
    o = f()
    assert epilogue_call(o=o, y=o + 4) == ALIAS


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="would launch on fake pointers")
def test_valid_arguments_reach_the_launch_without_gpu():
    """With no GPU present, valid arguments pass validation and the launch
    itself reports KDA_ERR_HIP (the library never falls back to the CPU)."""
    assert decode_call() == HIP
    assert chunk_call() == HIP
    assert dplr_call() == HIP
    assert bwd_call() == HIP
    assert prologue_call() == HIP
    assert epilogue_call() == HIP


def layer_fwd_call(**over):
    f = Fake()
    a = dict(xq=f(), xk=f(), xv=f(), xa=f(), xb=f(), wq=f(), wk=f(), wv=f(), A_log=f(), dtb=f(), s0=None, cu=None,
             N=1, T=100, H=2, d=64, o=f(), fs=f(), ws=f(), wsb=1 << 40, stream=None)
    a.update(over)
    P = ctypes.c_void_p
    return kda._load().kda_layer_chunk_fwd(*(P(a[x]) for x in ("xq", "xk", "xv", "xa", "xb", "wq", "wk", "wv",
                                                               "A_log", "dtb", "s0", "cu")),
                                           a["N"], a["T"], a["H"], a["d"], P(a["o"]), P(a["fs"]), P(a["ws"]),
                                           a["wsb"], P(a["stream"]))


def test_layer_fwd_workspace_and_validation():
    """The fused prologue + prefill: workspace = the bf16 forward's plus 2 x 64 x d
    bf16 per chunk-head (the exact path's q, k rows); host validation refuses
    every malformed call before any launch."""
    assert kda.layer_chunk_fwd_workspace_size(1, 4096, 32, 128) == 64 * 32 * (98816 + 2 * 64 * 128 * 2) + 256
    assert kda.layer_chunk_fwd_workspace_size(16, 135000, 32, 64) == (
        kda.workspace_size(16, 135000, 32, 64, 64) + ((135000 + 63 * 16) // 64) * 32 * 2 * 64 * 64 * 2)
    with pytest.raises(kda.KDAError):
        kda.layer_chunk_fwd_workspace_size(1, 10, 1, 96)
    assert layer_fwd_call(xq=None) == NULL
    assert layer_fwd_call(o=None) == NULL
    assert layer_fwd_call(N=2) == SHAPE  # no cu_seqlens
    assert layer_fwd_call(T=1 << 30, H=4) == SHAPE
    assert layer_fwd_call(d=96) == UNSUP
    f = Fake()
    assert layer_fwd_call(xq=f(2)) == ALIGN  # bf16 channel pairs
    assert layer_fwd_call(o=f(8)) == ALIGN
    assert layer_fwd_call(wsb=1024) == WORKSPACE
    assert layer_fwd_call(ws=f(128)) == WORKSPACE  # 256-byte aligned
    x = f()
    assert layer_fwd_call(xq=x, o=x + 64) == ALIAS
    y = f()
    assert layer_fwd_call(o=y, fs=y + 256) == ALIAS


def whole_layer_call(**over):
    f = Fake()
    a = dict(xq=f(), xk=f(), xv=f(), xa=f(), xb=f(), xg=f(), wq=f(), wk=f(), wv=f(), A_log=f(), dtb=f(), rw=f(),
             s0=None, cu=None, N=1, T=100, H=2, d=64, y=f(), fs=f(), ws=f(), wsb=1 << 40, stream=None)
    a.update(over)
    P = ctypes.c_void_p
    return kda._load().kda_layer_fwd(*(P(a[x]) for x in ("xq", "xk", "xv", "xa", "xb", "xg", "wq", "wk", "wv",
                                                         "A_log", "dtb", "rw", "s0", "cu")),
                                     a["N"], a["T"], a["H"], a["d"], P(a["y"]), P(a["fs"]), P(a["ws"]), a["wsb"],
                                     P(a["stream"]))


def test_whole_layer_workspace_and_validation():
    """kda_layer_fwd: workspace = kda_layer_chunk_fwd's plus the epilogue's region,
    rounded up to 256 bytes: with no device to query (as here) room for the
    operator's fp32 o, which the epilogue kernel reads (the GPU tests cover the
    fused epilogue's partial sums); host validation refuses every malformed
    call before any launch."""
    def up(x):
        return (x + 255) // 256 * 256

    for N, T, H, d in ((1, 4096, 32, 128), (1000, 1000, 2, 128), (16, 135000, 32, 64), (3, 0, 4, 64)):
        NC = (T + 63 * N) // 64
        extra = up(T * H * d * 4)
        assert kda.layer_fwd_workspace_size(N, T, H, d) == kda.layer_chunk_fwd_workspace_size(N, T, H, d) + extra
    with pytest.raises(kda.KDAError):
        kda.layer_fwd_workspace_size(1, 10, 1, 96)
    assert whole_layer_call(xg=None) == NULL
    assert whole_layer_call(rw=None) == NULL
    assert whole_layer_call(y=None) == NULL
    assert whole_layer_call(N=2) == SHAPE  # no cu_seqlens
    assert whole_layer_call(d=96) == UNSUP
    f = Fake()
    assert whole_layer_call(xg=f(4)) == ALIGN  # 4 channels per lane
    assert whole_layer_call(y=f(4)) == ALIGN
    assert whole_layer_call(rw=f(2)) == ALIGN
    assert whole_layer_call(wsb=kda.layer_chunk_fwd_workspace_size(1, 100, 2, 64)) == WORKSPACE
    x = f()
    assert whole_layer_call(xq=x, y=x + 64) == ALIAS
    g = f()
    assert whole_layer_call(xg=g, y=g + 8) == ALIAS
    fs = f()
    assert whole_layer_call(rw=fs + 64, fs=fs) == ALIAS
    w = f()
    assert whole_layer_call(ws=w, y=w + 1024) == ALIAS


def test_layer_decode_validation():
    """The convolution history and the one-token prologue refuse malformed calls
    before any launch."""
    f = Fake()
    P = ctypes.c_void_p
    lib = kda._load()

    def cs_call(**over):
        a = dict(xq=f(), xk=f(), xv=f(), cu=None, N=1, T=10, H=2, d=64, dt=BF16, cs=f())
        a.update(over)
        return lib.kda_layer_conv_state(P(a["xq"]), P(a["xk"]), P(a["xv"]), P(a["cu"]), a["N"], a["T"], a["H"],
                                        a["d"], a["dt"], P(a["cs"]), None)

    def dp_call(**over):
        a = dict(xq=f(), xk=f(), xv=f(), xa=f(), xb=f(), cs=f(), wq=f(), wk=f(), wv=f(), A_log=f(), dtb=f(), N=3,
                 H=2, d=64, dt=BF16, q=f(), k=f(), v=f(), la=f(), beta=f())
        a.update(over)
        return lib.kda_layer_decode_prologue(*(P(a[x]) for x in ("xq", "xk", "xv", "xa", "xb", "cs", "wq", "wk",
                                                                 "wv", "A_log", "dtb")),
                                             a["N"], a["H"], a["d"], a["dt"],
                                             *(P(a[x]) for x in ("q", "k", "v", "la", "beta")), None)

    assert cs_call(cs=None) == NULL
    assert cs_call(xq=None) == NULL
    assert cs_call(N=2) == SHAPE
    assert cs_call(d=96) == UNSUP
    assert cs_call(cs=f(2)) == ALIGN
    x = f()
    assert cs_call(xq=x, cs=x + 64) == ALIAS
    assert dp_call(N=0) == SHAPE
    assert dp_call(cs=None) == NULL
    assert dp_call(d=32) == UNSUP
    assert dp_call(cs=f(2)) == ALIGN
    assert dp_call(q=f(2)) == ALIGN
    y = f()
    assert dp_call(xq=y, cs=y + 64) == ALIAS  # the history is written in place
    z = f()
    assert dp_call(cs=z, q=z + 128) == ALIAS

    def ds_call(**over):
        a = dict(q=f(), k=f(), v=f(), la=f(), beta=f(), st=f(), xg=f(), w=f(), N=3, H=2, d=64, dt=BF16, y=f())
        a.update(over)
        return lib.kda_layer_decode_step(*(P(a[x]) for x in ("q", "k", "v", "la", "beta", "st", "xg", "w")),
                                         a["N"], a["H"], a["d"], a["dt"], P(a["y"]), None)

    assert ds_call(y=None) == NULL
    assert ds_call(xg=None) == NULL
    assert ds_call(w=None) == NULL
    assert ds_call(N=0) == SHAPE
    assert ds_call(H=-1) == SHAPE
    assert ds_call(d=96) == UNSUP
    assert ds_call(dt=7) == UNSUP
    assert ds_call(q=f(8)) == ALIGN      # 16 bytes
    assert ds_call(st=f(4)) == ALIGN
    assert ds_call(xg=f(2)) == ALIGN     # two bf16 elements
    assert ds_call(y=f(1)) == ALIGN
    assert ds_call(w=f(2)) == ALIGN      # 4 bytes
    u = f()
    assert ds_call(q=u, y=u + 256) == ALIAS
    w2 = f()
    assert ds_call(xg=w2, st=w2 + 512) == ALIAS
    v2 = f()
    assert ds_call(st=v2, y=v2 + 1024) == ALIAS


def test_noalloc_refuses_oversized_and_bad_shapes_on_host():
    """kda_chunk_fwd_noalloc refuses a call whose workspace exceeds its static
    scratch (KDA_ERR_WORKSPACE) and bad sizes (as kda_chunk_fwd does) before
    any device call, so these run without a GPU."""
    import ctypes as C
    lib = kda._load()
    f = Fake()
    def call(N, T, H, d, cu=None):
        return lib.kda_chunk_fwd_noalloc(f(), f(), f(), f(), f(), None, cu, N, T, H, d, d, BF16, BF16, F32,
                                         f(), f(), None)
    assert kda.workspace_size(1, 22 * 64, 32, 128, 128) > kda.NOALLOC_WORKSPACE_BYTES
    assert kda.workspace_size(1, 21 * 64, 32, 128, 128) <= kda.NOALLOC_WORKSPACE_BYTES
    assert call(1, 22 * 64, 32, 128) == WORKSPACE
    assert call(1, 1 << 20, 32, 128) == WORKSPACE
    assert call(0, 100, 32, 128) == SHAPE
    assert call(1, 100, 2, 96) == UNSUP
