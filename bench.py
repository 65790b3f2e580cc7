"""Benchmark of the KDA hot path on one MI355X.

One step = one chunkwise prefill call (per-chunk preparation, then the
inter-chunk state recursion with the chunk outputs fused in) on ``long-1m``,
the largest single-GPU workload: B=1, H=32, T=1,048,576 (16,384 chunks of 64
chained per head), dk=dv=128, bf16 inputs, fp32 initial/final state and fp32
output, inputs resident in HBM (synthetic, seeded; see kda_inputs). Timing
protocol: W untimed warm-up calls; then K calls, each preceded by a 512 MiB
write that flushes the 256 MB Infinity Cache (MALL), timed with HIP events on
the launch stream ("cold", the primary figure; median and min), then K calls
back to back ("warm"). The same protocol runs on ``prefill-4k`` and
``varlen-16`` (reported under "workloads"). The decode step (the remaining row
of the hot path) is timed on ``decode-256`` (256 sequences x 32 heads, fp32
states of 512 MiB, updated in place, 1000 steps). The general-DPLR comparison
operator and the layer around the operator are timed on prefill-4k, the
chunkwise backward on prefill-4k, varlen-16 and long-1m (in pieces). Prints ONE
JSON line.

    python bench.py [--steps K] [--warmup W] [--decode-steps S] [--headline-only] [--no-cpu-baseline]
                    [--no-dplr] [--no-bwd] [--no-layer] [--no-decode]

Profiling helpers (used to write the summaries under profiles/):
    python bench.py --copy-calibration MIB        # counter calibration kernel only
    python bench.py --report-trace DB             # kernel-trace database -> markdown
    python bench.py --report-pmc WORKLOAD FETCH_DB WRITE_DB CAL_FETCH_DB CAL_WRITE_DB CAL_BYTES
    python bench.py --report-counters DB [DB ...]  # any --pmc counters -> markdown, per kernel
    python bench.py --profile-set long-1m|prefill-4k   # one workload's dispatches per profile
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s + TFLOP/s (% MFMA peak); decode state GB/s (% HBM peak)"
PEAK_BF16 = 2.5e15       # dense bf16/fp16 MFMA, FLOP/s
PEAK_HBM = 8.0e12        # HBM3E, B/s
# per token-head, d = 128, chunk 64: flops of the chunkwise form (three d x d
# state products, five triangular chunk products, the forward substitution) and
# the operator's compulsory HBM bytes (its inputs and its output, once each)
FLOP_PER_TOKEN_HEAD = 140629
ALG_BYTES_PER_TOKEN_HEAD = 1538            # q,k,v,log_alpha bf16 + beta bf16 + o fp32
# this design's own pipeline traffic (its intermediates included), per token-head:
KERNEL_BYTES_PER_TOKEN_HEAD = {
    # reads q,k,v,log_alpha,beta; writes Q+,K-,-W (fp16 256 each), U (fp32 512),
    # A_qk (two fp16 planes 256), gamma 8
    "prep": 1026 + 1544,
    # with bf16 inputs the output is fused into the state recursion: reads -W, K-,
    # Q+ (256 each), U 512, A_qk 256, gamma 8; writes o (fp32 512)
    "recur": 1544 + 512,
}
# fp32 inputs (not benchmarked) run the unfused pair: the recursion reads -W, K-,
# U (fp32 512 each) and gamma 8 and writes h_n 1024 + V_new 512; the output reads
# Q+ 512, A_qk 256, h_n 1024, V_new 512 and writes o 512
KERNEL_SYMBOL = {"prep": "prep_kernel", "recur": "recur_kernel", "decode": "decode_kernel",
                 "dplr_prep": "dplr_prep_kernel", "dplr_recur": "recur_kernel",
                 "bwd_fwd_prep": "prep_kernel", "bwd_fwd_recur": "recur_kernel",
                 "bwd_prep": "bwd_prep_kernel", "bwd_recur": "recur_kernel", "bwd_local": "bwd_local_kernel",
                 "layer_prologue": "layer_prologue_kernel", "layer_epilogue": "layer_epilogue_kernel",
                 "layer_prep": "prep_kernel", "layer_recur": "recur_kernel", "layer_decode": "decode_kernel"}
# each kernel's source file and the library headers it includes (with kda_common.h, which all do)
_PREP = ("kda_prep.hip", "kda_prep_util.h", "kda_layer_util.h")
_RECUR = ("kda_recur.hip", "kda_prep_util.h", "kda_layer_util.h")
_DECODE = ("kda_decode.hip", "kda_layer_util.h")
KERNEL_SOURCE = {"prep": _PREP, "recur": _RECUR, "decode": _DECODE,
                 "dplr_prep": ("kda_dplr_prep.hip", "kda_prep_util.h"), "dplr_recur": _RECUR,
                 "bwd_fwd_prep": _PREP, "bwd_fwd_recur": _RECUR,
                 "bwd_prep": ("kda_bwd.hip", "kda_prep_util.h"), "bwd_recur": _RECUR,
                 "bwd_local": ("kda_bwd.hip", "kda_prep_util.h"),
                 "layer_prologue": ("kda_layer.hip", "kda_layer_util.h"),
                 "layer_epilogue": ("kda_layer.hip", "kda_layer_util.h"),
                 "layer_prep": _PREP, "layer_recur": _RECUR, "layer_decode": _DECODE}


def kernel_key(short_name: str):
    """Which of this library's kernels a demangled name (arguments stripped) is.
    The template arguments tell the instantiations apart: the preparation's
    last two are fp32 factors (the backward's forward recompute) and the fused
    layer prologue; the state
    recursion's are <D, fp32 factors, fused output, fp32 output, DPLR chain,
    added per-chunk term (the backward's state-gradient recursion), fused layer
    epilogue>."""
    if "<" not in short_name:
        return None
    sym, args = short_name.split("<", 1)
    args = [x.strip() for x in args.rstrip(">").split(",")]
    flag = lambda i: len(args) > i and args[i] == "true"
    if sym == "recur_kernel":
        if flag(6):
            return "layer_recur"
        if flag(5):
            return "bwd_recur"
        if flag(4):
            return "dplr_recur"
        return "bwd_fwd_recur" if flag(1) else "recur"
    if sym == "prep_kernel":  # <D, TIn, TG, fp32 factors, fused layer prologue>
        if flag(4):
            return "layer_prep"
        return "bwd_fwd_prep" if flag(3) else "prep"
    if sym == "decode_kernel":  # <D, TIn, TG, fp32 o, fused layer epilogue>
        return "layer_decode" if flag(4) else "decode"
    for key in ("dplr_prep", "bwd_prep", "bwd_local", "layer_prologue", "layer_epilogue"):
        if sym == KERNEL_SYMBOL[key]:
            return key
    return None


def hip_runtime():
    for name in ("libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"):
        try:
            lib = ctypes.CDLL(name)
            lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            return lib
        except OSError:
            continue
    raise RuntimeError("libamdhip64.so not found")


class Events:
    def __init__(self, hip, n):
        self.hip = hip
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e.value)

    def record(self, i, stream):
        if self.hip.hipEventRecord(ctypes.c_void_p(self.ev[i]), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b):
        self.hip.hipEventSynchronize(ctypes.c_void_p(self.ev[b]))
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(self.ev[a]),
                                        ctypes.c_void_p(self.ev[b])) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    src = KERNEL_SOURCE[kernel]
    for f in (*(src if isinstance(src, tuple) else (src,)), "kda_common.h"):
        with open(os.path.join(ROOT, "gated_delta_rule_41_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str, workload: str = "prefill-4k"):
    """HBM bytes per launch from committed rocprofv3 --pmc counters, if they were
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha") != source_sha(kernel):
        return None
    return rec.get("bytes_per_launch")


class Flusher:
    """Writes a scratch buffer larger than the 256 MB Infinity Cache (MALL), on
    torch's current stream, so the next call starts with cold caches."""

    def __init__(self, mib: int, dev):
        import torch
        self.mib = mib
        self.buf = torch.empty(mib * (1 << 20) // 4, dtype=torch.float32, device=dev) if mib > 0 else None

    def __call__(self):
        if self.buf is not None:
            self.buf.fill_(1.0)


def _stats(xs):
    xs = sorted(xs)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    return round(med, 5), round(xs[0], 5)


def time_prefill(kda, case, steps, warmup, hip, stream, flush):
    """The prefill timing protocol: ``warmup`` untimed calls; then ``steps``
    calls each preceded by a cache flush ("cold"), with HIP events recorded by
    the library on the launch stream before the preparation kernel, between it
    and the recursion, and after the recursion (its output is fused with bf16
    inputs); the wall clock brackets these steps (flushes included) between two
    synchronizations; then ``steps`` calls back to back, each between two events
    ("warm"). Returns a dict of per-call times (ms) and the outputs."""
    import torch
    dev = case.q.device
    ws = torch.empty(kda.workspace_size(case.N, case.T_total, case.H, case.dk, case.dv, case.q.dtype),
                     dtype=torch.uint8, device=dev)
    o = torch.empty(case.T_total, case.H, case.dv, dtype=torch.float32, device=dev)
    fs = torch.empty(case.N, case.H, case.dk, case.dv, dtype=torch.float32, device=dev)

    def call(events=None):
        kda.chunk_fwd(case.q, case.k, case.v, case.log_alpha, case.beta, case.initial_state,
                      case.cu_seqlens, o=o, final_state=fs, workspace=ws, events=events)

    for _ in range(warmup):
        call()
    # the flush kernel and the event-recording path run once before the timed
    # loop (the first launch of a kernel pays its module load on the host)
    flush()
    ev0 = Events(hip, 4)
    call(events=ev0.ev)
    torch.cuda.synchronize()
    ev0.close()
    ev = Events(hip, 4 * steps)
    t0 = time.perf_counter()
    for s_ in range(steps):
        flush()
        call(events=ev.ev[4 * s_:4 * s_ + 4])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    res = {"wall_ms": wall_ms, "cold": [], "prep": [], "recur": []}
    for s_ in range(steps):
        b = 4 * s_
        res["cold"].append(ev.ms(b, b + 3))
        res["prep"].append(ev.ms(b, b + 1))
        res["recur"].append(ev.ms(b + 1, b + 3))  # state recursion with the fused output
    ev.close()
    ev = Events(hip, 2 * steps)
    for s_ in range(steps):
        ev.record(2 * s_, stream)
        call()
        ev.record(2 * s_ + 1, stream)
    torch.cuda.synchronize()
    res["warm"] = [ev.ms(2 * s_, 2 * s_ + 1) for s_ in range(steps)]
    ev.close()
    del ws
    return res, o, fs


def prefill_report(case, res):
    """Throughput and roofline figures of one prefill workload from its timings."""
    TH = case.T_total * case.H
    flops = FLOP_PER_TOKEN_HEAD * TH
    states = (2 if case.initial_state is not None else 1) * case.N * case.H * case.dk * case.dv * 4
    alg_bytes = ALG_BYTES_PER_TOKEN_HEAD * TH + states
    ceiling = min(PEAK_BF16, flops / alg_bytes * PEAK_HBM)
    cold_med, cold_min = _stats(res["cold"])
    warm_med, warm_min = _stats(res["warm"])
    kern = {"prep": _stats(res["prep"])[0], "recur": _stats(res["recur"])[0]}
    dom = max(kern, key=kern.get)
    achieved = alg_bytes / (kern[dom] * 1e-3)
    rep = {"T_total": case.T_total, "N": case.N, "H": case.H,
           "cold_ms_median": cold_med, "cold_ms_min": cold_min, "warm_ms_median": warm_med,
           "warm_ms_min": warm_min, "tokens_per_s": round(case.T_total / (cold_med * 1e-3), 1),
           "tflops": round(flops / (cold_med * 1e-3) / 1e12, 2),
           "mfma_peak_frac": round(flops / (cold_med * 1e-3) / PEAK_BF16, 4),
           "alg_roofline_frac": round(flops / (cold_med * 1e-3) / ceiling, 4),
           "alg_ceiling_tflops": round(ceiling / 1e12, 1), "alg_bytes": alg_bytes,
           "kernel_ms_cold_median": kern}
    roof = {"kernel": KERNEL_SYMBOL[dom], "bound": "hbm", "achieved": round(achieved / 1e9, 1),
            "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": round(achieved / PEAK_HBM, 4),
            "avg_launch_ms": kern[dom], "alg_bytes_per_launch": alg_bytes}
    return rep, roof, dom


def time_dplr(kda, case, steps, warmup):
    """Whole-call time of the general-DPLR prefill (its two kernels) on the
    stream the binding launches on, with torch events (torch's current stream)."""
    import torch
    dev = case.q.device
    ws = torch.empty(kda.dplr_workspace_size(case.N, case.T_total, case.H, case.dk, case.dv),
                     dtype=torch.uint8, device=dev)
    o = torch.empty(case.T_total, case.H, case.dv, dtype=torch.float32, device=dev)
    fs = torch.empty(case.N, case.H, case.dk, case.dv, dtype=torch.float32, device=dev)

    def call():
        kda.dplr_chunk_fwd(case.q, case.k, case.v, case.a, case.b, case.log_alpha, case.initial_state,
                           case.cu_seqlens, o=o, final_state=fs, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, o, fs


def bwd_pieces(case):
    """Pieces the backward runs in with the default workspace: one while the
    chunk slots x heads fit 65536, else slots of floor(65536 / H) each."""
    nc = (case.T_total + 63 * case.N) // 64 if case.cu_seqlens is not None else (case.T_total + 63) // 64
    if nc * case.H <= 65536:
        return 1
    per = max(65536 // case.H, 1)
    return -(-nc // per)


def time_bwd(kda, case, steps, warmup):
    """Whole-call time of the chunkwise backward (the fp32 forward recompute,
    the operand preparation, the reverse state-gradient recursion and the local
    adjoints; in pieces, the checkpoint forward first), torch events on torch's
    current stream, which the binding launches on."""
    import torch
    dev = case.q.device
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    d_o = torch.randn(case.T_total, case.H, case.dv, generator=g, device=dev)
    d_fin = torch.randn(case.N, case.H, case.dk, case.dv, generator=g, device=dev) * 0.1
    ws = torch.empty(kda.bwd_workspace_size(case.N, case.T_total, case.H, case.dk, case.dv),
                     dtype=torch.uint8, device=dev)
    shapes = {"dq": (case.T_total, case.H, case.dk), "dk": (case.T_total, case.H, case.dk),
              "dv": (case.T_total, case.H, case.dv), "dlog_alpha": (case.T_total, case.H, case.dk),
              "dbeta": (case.T_total, case.H), "dinitial_state": (case.N, case.H, case.dk, case.dv)}
    outs = {k_: torch.empty(*s_, dtype=torch.float32, device=dev) for k_, s_ in shapes.items()}

    def call():
        return kda.chunk_bwd(case.q, case.k, case.v, case.log_alpha, case.beta, d_o, case.initial_state,
                             case.cu_seqlens, d_fin, workspace=ws, out=outs)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, ws.numel()


def time_layer(kda, lc, steps, warmup, hip, stream):
    """The layer path around the operator on one workload: prologue, the
    operator, epilogue. Outputs and the operator's workspace are allocated once;
    the three calls go straight through the C ABI (so no host work sits between
    the launches) and HIP events on the launch stream bracket each part. Returns ms per prologue, operator call, epilogue and whole layer."""
    import torch
    lib = kda._load()
    T, H, d = lc.xq.shape
    dev = lc.xq.device
    q, k, v, la = (torch.empty(T, H, d, dtype=lc.xq.dtype, device=dev) for _ in range(4))
    beta = torch.empty(T, H, dtype=lc.xq.dtype, device=dev)
    o = torch.empty(T, H, d, dtype=torch.float32, device=dev)
    N = 1 if lc.cu_seqlens is None else lc.cu_seqlens.numel() - 1
    fs = torch.empty(N, H, d, d, dtype=torch.float32, device=dev)
    ws = torch.empty(kda.workspace_size(N, T, H, d, d, q.dtype), dtype=torch.uint8, device=dev)
    y = torch.empty(T, H, d, dtype=lc.xg.dtype, device=dev)
    P = ctypes.c_void_p

    def ptr(t):
        return None if t is None else P(t.data_ptr())
    dtc = kda.KDA_BF16 if lc.xq.dtype == torch.bfloat16 else kda.KDA_F32
    pro_args = (*(ptr(t) for t in (lc.xq, lc.xk, lc.xv, lc.xa, lc.xb, lc.wq, lc.wk, lc.wv, lc.A_log,
                                   lc.dt_bias, lc.cu_seqlens)),
                N, T, H, d, dtc, *(ptr(t) for t in (q, k, v, la, beta)), P(stream))
    epi_args = (ptr(o), ptr(lc.xg), ptr(lc.rms_w), T, H, d, dtc, ptr(y), P(stream))
    op_args = (*(ptr(t) for t in (q, k, v, la, beta, lc.initial_state, lc.cu_seqlens)), N, T, H, d, d, dtc, dtc,
               kda.KDA_F32, ptr(o), ptr(fs), ptr(ws), ws.numel(), P(stream))
    fws = torch.empty(kda.layer_chunk_fwd_workspace_size(N, T, H, d), dtype=torch.uint8, device=dev)
    fused_args = (*(ptr(t) for t in (lc.xq, lc.xk, lc.xv, lc.xa, lc.xb, lc.wq, lc.wk, lc.wv, lc.A_log, lc.dt_bias,
                                     lc.initial_state, lc.cu_seqlens)),
                  N, T, H, d, ptr(o), ptr(fs), ptr(fws), fws.numel(), P(stream))

    def step(ev=None, b=0):
        if ev is not None:
            ev.record(b, stream)
        if lib.kda_layer_prologue(*pro_args) != 0:
            raise RuntimeError("kda_layer_prologue failed")
        if ev is not None:
            ev.record(b + 1, stream)
        if lib.kda_chunk_fwd(*op_args) != 0:
            raise RuntimeError("kda_chunk_fwd failed")
        if ev is not None:
            ev.record(b + 2, stream)
        if lib.kda_layer_epilogue(*epi_args) != 0:
            raise RuntimeError("kda_layer_epilogue failed")
        if ev is not None:
            ev.record(b + 3, stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # the whole layer back to back, events only around the loop
    ev = Events(hip, 2)
    ev.record(0, stream)
    for _ in range(steps):
        step()
    ev.record(1, stream)
    torch.cuda.synchronize()
    out = {"layer": ev.ms(0, 1) / steps, "prologue": 0.0, "operator": 0.0, "epilogue": 0.0}
    ev.close()
    # the parts, each bracketed by its own events (which add a little idle time)
    ev = Events(hip, 4 * steps)
    for s_ in range(steps):
        step(ev, 4 * s_)
    torch.cuda.synchronize()
    for s_ in range(steps):
        b = 4 * s_
        out["prologue"] += ev.ms(b, b + 1) / steps
        out["operator"] += ev.ms(b + 1, b + 2) / steps
        out["epilogue"] += ev.ms(b + 2, b + 3) / steps
    ev.close()
    # the fused path (bf16): prologue inside the chunk preparation, then the epilogue
    if lc.xq.dtype == torch.bfloat16:
        def fused_step():
            if lib.kda_layer_chunk_fwd(*fused_args) != 0:
                raise RuntimeError("kda_layer_chunk_fwd failed")
            if lib.kda_layer_epilogue(*epi_args) != 0:
                raise RuntimeError("kda_layer_epilogue failed")
        for _ in range(warmup):
            fused_step()
        torch.cuda.synchronize()
        ev = Events(hip, 2)
        ev.record(0, stream)
        for _ in range(steps):
            fused_step()
        ev.record(1, stream)
        torch.cuda.synchronize()
        out["fused_layer"] = ev.ms(0, 1) / steps
        ev.close()
        # the whole layer in one call: the epilogue inside the recursion's output stage too
        wws = torch.empty(kda.layer_fwd_workspace_size(N, T, H, d), dtype=torch.uint8, device=dev)
        whole_args = (*(ptr(t) for t in (lc.xq, lc.xk, lc.xv, lc.xa, lc.xb, lc.xg, lc.wq, lc.wk, lc.wv, lc.A_log,
                                         lc.dt_bias, lc.rms_w, lc.initial_state, lc.cu_seqlens)),
                      N, T, H, d, ptr(y), ptr(fs), ptr(wws), wws.numel(), P(stream))

        def whole_step():
            if lib.kda_layer_fwd(*whole_args) != 0:
                raise RuntimeError("kda_layer_fwd failed")
        for _ in range(warmup):
            whole_step()
        torch.cuda.synchronize()
        ev = Events(hip, 2)
        ev.record(0, stream)
        for _ in range(steps):
            whole_step()
        ev.record(1, stream)
        torch.cuda.synchronize()
        out["one_call_layer"] = ev.ms(0, 1) / steps
        ev.close()
        del wws
    return out


def time_layer_decode(kda, ki, steps, warmup, hip, stream, N=256, H=32, d=128):
    """The layer's decode step at decode-256 size (one bf16 token per sequence):
    decode prologue (history in place), kda_decode_step (fp32 state in place),
    epilogue, all through the C ABI between two events around the loop; then
    the same with kda_layer_decode_step (the epilogue fused into the decode
    kernel) in place of the last two. Returns ms per step of each."""
    import torch
    lib = kda._load()
    lc = ki.make_layer("decode-256", "cuda:0", lengths=[1] * N, H=H, d=d, s0_std=0.0)  # one token's pre-activations each
    dev = lc.xq.device
    cs = torch.zeros(N, H, 3, 3, d, dtype=torch.bfloat16, device=dev)
    state = 0.02 * torch.randn(N, H, d, d, device=dev)
    q, k, v, la = (torch.empty(N, H, d, dtype=torch.bfloat16, device=dev) for _ in range(4))
    beta = torch.empty(N, H, dtype=torch.bfloat16, device=dev)
    o = torch.empty(N, H, d, dtype=torch.float32, device=dev)
    y = torch.empty(N, H, d, dtype=torch.bfloat16, device=dev)
    P = ctypes.c_void_p
    bf = kda.KDA_BF16

    def ptr(t):
        return P(t.data_ptr())
    pro = (*(ptr(t) for t in (lc.xq, lc.xk, lc.xv, lc.xa, lc.xb, cs, lc.wq, lc.wk, lc.wv, lc.A_log, lc.dt_bias)),
           N, H, d, bf, *(ptr(t) for t in (q, k, v, la, beta)), P(stream))
    dec = (*(ptr(t) for t in (q, k, v, la, beta, state)), N, H, d, d, bf, bf, kda.KDA_F32, ptr(o), P(stream))
    epi = (ptr(o), ptr(lc.xg), ptr(lc.rms_w), N, H, d, bf, ptr(y), P(stream))

    fused = (*(ptr(t) for t in (q, k, v, la, beta, state, lc.xg, lc.rms_w)), N, H, d, bf, ptr(y), P(stream))

    def step():
        if lib.kda_layer_decode_prologue(*pro) != 0 or lib.kda_decode_step(*dec) != 0 or \
                lib.kda_layer_epilogue(*epi) != 0:
            raise RuntimeError("layer decode step failed")

    def step_fused():
        if lib.kda_layer_decode_prologue(*pro) != 0 or lib.kda_layer_decode_step(*fused) != 0:
            raise RuntimeError("fused layer decode step failed")
    res = []
    for fn in (step, step_fused):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = Events(hip, 2)
        ev.record(0, stream)
        for _ in range(steps):
            fn()
        ev.record(1, stream)
        torch.cuda.synchronize()
        res.append(ev.ms(0, 1) / steps)
        ev.close()
    return res[0], res[1]


def time_decode(kda, dec, steps, warmup, hip, stream):
    import torch
    state = dec["state"]
    o = torch.empty(state.shape[0], state.shape[1], state.shape[3], dtype=torch.float32,
                    device=state.device)
    n_in = dec["q"].shape[0]
    for s in range(warmup):
        j = s % n_in
        kda.decode_step(dec["q"][j], dec["k"][j], dec["v"][j], dec["log_alpha"][j], dec["beta"][j], state, o=o)
    torch.cuda.synchronize()
    ev = Events(hip, 2)
    ev.record(0, stream)
    for s in range(steps):
        j = s % n_in
        kda.decode_step(dec["q"][j], dec["k"][j], dec["v"][j], dec["log_alpha"][j], dec["beta"][j], state, o=o)
    ev.record(1, stream)
    torch.cuda.synchronize()
    ms = ev.ms(0, 1) / steps
    ev.close()
    return ms


def copy_bandwidth(hip, stream, mib: int = 1024, reps: int = 20):
    """Achievable HBM rate of a plain streaming kernel on this GPU (y = x * 1 over
    ``mib`` MiB of fp32, read + write), as a measured reference beside the
    datasheet peak."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(3):
        torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    ev = Events(hip, 2)
    ev.record(0, stream)
    for _ in range(reps):
        torch.mul(x, 1.0, out=y)
    ev.record(1, stream)
    torch.cuda.synchronize()
    ms = ev.ms(0, 1) / reps
    ev.close()
    del x, y
    return 2 * 4 * n / (ms * 1e-3) / 1e9


def machine_peaks(hip, stream):
    """Achievable rates of this GPU, measured beside the datasheet peaks by the
    probes in libkda_probe.so: a bf16 matrix-core loop (1,024 workgroups of four
    waves, eight independent accumulators each, 16x16x32 products back to back)
    and a streaming copy (16-byte nontemporal loads and stores over 2 GiB each
    way). Both run on the launch stream between HIP events; the best of 5 calls
    after 2 warm-ups is reported."""
    import torch
    path = os.path.join(ROOT, "gated_delta_rule_41_amd", "libkda_probe.so")
    lib = ctypes.CDLL(path)
    lib.kda_probe_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.kda_probe_mfma_bf16.restype = ctypes.c_int32
    lib.kda_probe_mfma_bf16_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.kda_probe_mfma_bf16_flops.restype = ctypes.c_double
    lib.kda_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
    lib.kda_probe_copy.restype = ctypes.c_int32

    def best(call, reps=5, warm=2):
        for _ in range(warm):
            call()
        torch.cuda.synchronize()
        ev = Events(hip, 2 * reps)
        for r in range(reps):
            ev.record(2 * r, stream)
            call()
            ev.record(2 * r + 1, stream)
        torch.cuda.synchronize()
        t = min(ev.ms(2 * r, 2 * r + 1) for r in range(reps))
        ev.close()
        return t

    n_wg, iters = 1024, 20000
    sink = torch.empty(n_wg * 4, dtype=torch.float32, device="cuda:0")

    def mfma():
        if lib.kda_probe_mfma_bf16(n_wg, iters, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("kda_probe_mfma_bf16 failed")
    ms = best(mfma)
    tflops = lib.kda_probe_mfma_bf16_flops(n_wg, iters) / (ms * 1e-3) / 1e12
    nbytes = 2 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")

    def copy():
        if lib.kda_probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes,
                              ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("kda_probe_copy failed")
    cms = best(copy)
    del src, dst, sink
    torch.cuda.empty_cache()
    probe_gbps = 2 * nbytes / (cms * 1e-3) / 1e9
    torch_gbps = copy_bandwidth(hip, stream)
    copy_gbps = max(probe_gbps, torch_gbps)
    return {"bf16_mfma_tflops": round(tflops, 1), "bf16_mfma_frac_of_datasheet": round(tflops * 1e12 / PEAK_BF16, 4),
            "copy_GBps": round(copy_gbps, 1), "copy_frac_of_datasheet": round(copy_gbps * 1e9 / PEAK_HBM, 4),
            "copy_probe_GBps": round(probe_gbps, 1), "torch_copy_GBps": round(torch_gbps, 1),
            "probes": "bf16 16x16x32 MFMA loop, 1024 workgroups x 4 waves x 8 accumulators; copy = the faster of "
                      "a nontemporal 16-byte copy of 2 GiB and torch's y = x * 1 over 1 GiB (bytes read + written)"}


def cpu_baseline(host, T, H, dk, rec_pos, threads):
    """The oracle (fp64 token recurrence, OpenMP over (head, column block)) on
    the host cores, on the headline workload's own inputs copied to the host:
    every head over the whole sequence, the output kept at ``rec_pos`` only."""
    import oracle
    t0 = time.perf_counter()
    _, S_ref, o_rec = oracle.recurrence(*host, None, want_o=False, rec_pos=rec_pos, col_blocks=1,
                                        threads=threads)
    dt = time.perf_counter() - t0
    return {"value": T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"long-1m in full (T={T}, all {H} heads, d={dk}, fp64 token recurrence; final states "
                      f"and o at {len(rec_pos)} sampled positions kept), {dt:.1f} s wall"}, S_ref, o_rec


def cpu_single_thread(case, heads=None):
    """The oracle on one host thread, on a bounded sample of prefill-4k (the
    first ``heads`` heads, default all, over the whole sequence), as tokens/s
    of all heads."""
    import oracle
    heads = case.H if heads is None else heads
    host = [t.cpu() for t in (case.q, case.k, case.v, case.log_alpha, case.beta, case.initial_state)]
    t0 = time.perf_counter()
    oracle.recurrence(*host, None, heads=list(range(heads)), want_o=True, col_blocks=1, threads=1)
    dt = time.perf_counter() - t0
    return {"value": case.T_total * heads / case.H / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"prefill-4k, {heads} of {case.H} heads over T={case.T_total}, one thread, {dt:.1f} s wall"}


def environment():
    """What ran: GPU, ROCm, torch, host CPU, and the library's source hash (and
    the git commit when the tree has one)."""
    import torch
    env = {}
    try:
        p = torch.cuda.get_device_properties(0)
        env["gpu"] = p.name
        env["gpu_arch"] = getattr(p, "gcnArchName", None)
        env["gpu_cus"] = p.multi_processor_count
    except Exception:  # pragma: no cover
        pass
    for f in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        if os.path.exists(f):
            env["rocm"] = open(f).read().strip()
            break
    env["torch"] = torch.__version__
    env["torch_hip"] = getattr(torch.version, "hip", None)
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                env["host_cpu"] = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    env["host_threads_visible"] = os.cpu_count()
    h = hashlib.sha256()
    for d in ("gated_delta_rule_41_amd/csrc", "include"):
        for f in sorted(os.listdir(os.path.join(ROOT, d))):
            with open(os.path.join(ROOT, d, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    env["library_source_sha16"] = h.hexdigest()[:16]
    try:
        import subprocess
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=10)
        env["git_commit"] = r.stdout.strip() if r.returncode == 0 else None
    except Exception:  # pragma: no cover
        env["git_commit"] = None
    return env


def copy_calibration(mib: int = 512, reps: int = 5):
    """A plain streaming kernel of known size (y = x * 1, fp32, ``mib`` MiB read and
    ``mib`` MiB written per launch) whose FETCH_SIZE / WRITE_SIZE counters give
    the scale from those counters to bytes. Run in a process of its own so that
    it is the only multiply kernel the profiler sees."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(reps):
        torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": 4 * n, "bytes_written": 4 * n, "reps": reps}}))
    return 0


def _rocpd(path):
    import sqlite3
    return sqlite3.connect(f"file:{path}?mode=ro", uri=True).cursor()


def _short(name: str) -> str:
    base = name.split("(")[0]
    return base.replace("void ", "").replace("kda::", "")


def report_trace(db: str) -> int:
    """Markdown table of this library's kernels from a rocprofv3 --kernel-trace
    database: dispatch count and duration statistics (microseconds)."""
    cur = _rocpd(db)
    rows = cur.execute("select name, count(*), avg(duration), min(duration), max(duration), sum(duration) "
                       "from kernels where name like '%kda::%' group by name order by sum(duration) desc").fetchall()
    print("| kernel | calls | avg us | min us | max us | total us |")
    print("|---|---|---|---|---|---|")
    for name, n, avg, mn, mx, tot in rows:
        print(f"| `{_short(name)}` | {n} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} | {tot / 1e3:.1f} |")
    return 0


def _counter_avg(db: str, counter: str, like: str):
    cur = _rocpd(db)
    return cur.execute("select kernel_name, count(*), avg(value) from counters_collection "
                       "where counter_name = ? and kernel_name like ? group by kernel_name",
                       (counter, like)).fetchall()


def report_pmc(workload: str, fetch_db: str, write_db: str, cal_fetch_db: str, cal_write_db: str,
               cal_bytes: int) -> int:
    """HBM traffic per launch of each library kernel from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch, one rocprofv3 --pmc run each), each scaled by
    what the same counter reads for the calibration copy kernel of known size.
    Writes profiles/pmc_<kernel>_<workload>.json (the decode kernel's as
    decode-256; read back by the roofline report while the kernel source is
    unchanged) and prints a markdown table."""
    cf = _counter_avg(cal_fetch_db, "FETCH_SIZE", "%MulFunctor%")
    cw = _counter_avg(cal_write_db, "WRITE_SIZE", "%MulFunctor%")
    if not cf or not cw:
        print("calibration kernel not found in the counter databases", file=sys.stderr)
        return 1
    f_fetch = cal_bytes / (cf[0][2] * 1024.0)
    f_write = cal_bytes / (cw[0][2] * 1024.0)
    fe = {_short(n): (c, v) for n, c, v in _counter_avg(fetch_db, "FETCH_SIZE", "%kda::%")}
    wr = {_short(n): (c, v) for n, c, v in _counter_avg(write_db, "WRITE_SIZE", "%kda::%")}
    print(f"calibration (y = x*1 over {cal_bytes >> 20} MiB): FETCH_SIZE {cf[0][2]:.0f} KiB -> scale {f_fetch:.4f}; "
          f"WRITE_SIZE {cw[0][2]:.0f} KiB -> scale {f_write:.4f}\n")
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch (scaled) |")
    print("|---|---|---|---|---|")
    for name in sorted(fe):
        if name not in wr:
            continue
        kern = kernel_key(name)
        b = fe[name][1] * 1024 * f_fetch + wr[name][1] * 1024 * f_write
        print(f"| `{name}` | {fe[name][0]} | {fe[name][1]:.0f} | {wr[name][1]:.0f} | {b:.4g} |")
        if kern is None:
            continue
        wl = "decode-256" if kern in ("decode", "layer_decode") else workload
        rec = {"kernel": name, "workload": wl, "source_sha": source_sha(kern),
               "fetch_kib": fe[name][1], "write_kib": wr[name][1],
               "fetch_scale": f_fetch, "write_scale": f_write, "bytes_per_launch": round(b)}
        with open(os.path.join(ROOT, "profiles", f"pmc_{kern}_{wl}.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
    return 0


def report_counters(*dbs: str) -> int:
    """Markdown table of every counter in one or more rocprofv3 --pmc databases,
    averaged per dispatch of each of this library's kernels, with the derived
    ratios used in the kernel analysis when their counters are present."""
    rows = {}
    for db in dbs:
        cur = _rocpd(db)
        for name, counter, n, val in cur.execute(
                "select kernel_name, counter_name, count(*), avg(value) from counters_collection "
                "where kernel_name like '%kda::%' group by kernel_name, counter_name").fetchall():
            rows.setdefault(_short(name), {})[counter] = (n, val)
    counters = sorted({c for r in rows.values() for c in r})
    print("| kernel | " + " | ".join(counters) + " |")
    print("|---|" + "---|" * len(counters))
    for name in sorted(rows):
        vals = [f"{rows[name][c][1]:.4g}" if c in rows[name] else "" for c in counters]
        print(f"| `{name}` | " + " | ".join(vals) + " |")
    print()
    for name in sorted(rows):
        r = {c: v for c, (_, v) in rows[name].items()}
        parts = []
        if "SQ_WAIT_INST_ANY" in r and "SQ_WAVE_CYCLES" in r and r["SQ_WAVE_CYCLES"]:
            parts.append(f"wave cycles waiting on an instruction's inputs {r['SQ_WAIT_INST_ANY'] / r['SQ_WAVE_CYCLES']:.1%}")
        if "SQ_WAIT_ANY" in r and "SQ_WAVE_CYCLES" in r and r["SQ_WAVE_CYCLES"]:
            parts.append(f"waiting on anything {r['SQ_WAIT_ANY'] / r['SQ_WAVE_CYCLES']:.1%}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in r and "GRBM_GUI_ACTIVE" in r and r["GRBM_GUI_ACTIVE"]:
            # MFMA busy cycles are summed over the 1,024 SIMDs; GRBM_GUI_ACTIVE
            # over the 8 XCDs (8 x the kernel's elapsed cycles)
            simd_cycles = r["GRBM_GUI_ACTIVE"] / 8 * 1024
            parts.append(f"matrix cores busy {r['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cycles:.1%} of SIMD cycles")
        if "SQ_LDS_BANK_CONFLICT" in r and "SQ_ACTIVE_INST_LDS" in r and r["SQ_ACTIVE_INST_LDS"]:
            parts.append(f"LDS bank-conflict cycles per active LDS cycle "
                         f"{r['SQ_LDS_BANK_CONFLICT'] / r['SQ_ACTIVE_INST_LDS']:.3f}")
        if "TCC_HIT_sum" in r and "TCC_MISS_sum" in r and (r["TCC_HIT_sum"] + r["TCC_MISS_sum"]):
            parts.append(f"L2 hit rate {r['TCC_HIT_sum'] / (r['TCC_HIT_sum'] + r['TCC_MISS_sum']):.1%}")
        if "SQ_WAVES" in r:
            parts.append(f"waves {r['SQ_WAVES']:.4g}")
        if parts:
            print(f"- `{name}`: " + "; ".join(parts))
    return 0


def main(argv=None):
    if argv is None:
        argv = sys.argv[1:]
    if argv[:1] == ["--report-trace"]:
        return report_trace(argv[1])
    if argv[:1] == ["--report-counters"]:
        return report_counters(*argv[1:])
    if argv[:1] == ["--report-pmc"]:
        return report_pmc(argv[1], argv[2], argv[3], argv[4], argv[5], int(argv[6]))
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5, help="timed calls per protocol leg")
    ap.add_argument("--warmup", type=int, default=2, help="untimed calls first")
    ap.add_argument("--flush-mib", type=int, default=512, help="cache flush written before each cold call")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--headline-only", action="store_true",
                    help="only the long-1m prefill (for profiling runs)")
    ap.add_argument("--profile-set", choices=["long-1m", "prefill-4k"], default=None,
                    help="profiling runs: only the long-1m prefill, or only the prefill-4k-sized legs (prefill-4k, "
                         "DPLR, backward, layer) and decode-256, so each profile holds one workload's dispatches")
    ap.add_argument("--workloads", default="prefill-4k,varlen-16",
                    help="prefill workloads timed beside the headline (same protocol)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-machine-peaks", action="store_true",
                    help="skip the measured MFMA and copy rates (libkda_probe.so)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-dplr", action="store_true", help="skip the general-DPLR comparison")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward")
    ap.add_argument("--no-layer", action="store_true", help="skip the layer prologue/epilogue")
    ap.add_argument("--no-layer-decode", action="store_true",
                    help="skip the layer's decode step (its epilogue launches are far smaller than the prefill's, "
                         "and a profile averages them together)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run the counter calibration copy kernel over MIB MiB")
    args = ap.parse_args(argv)
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration)
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU sharding is not implemented", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import gated_delta_rule_41_amd as kda
    import kda_inputs as ki

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 3
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hip = hip_runtime()
    stream = torch.cuda.current_stream(dev).cuda_stream
    flush = Flusher(args.flush_mib, dev)
    if args.profile_set == "long-1m":
        args.headline_only = True
    if args.headline_only:
        args.no_cpu_baseline = args.no_decode = args.no_dplr = args.no_bwd = args.no_layer = True
        args.no_machine_peaks = True
        args.workloads = ""
    t_start = time.perf_counter()
    if args.profile_set == "prefill-4k":
        args.no_cpu_baseline = True
        args.no_layer_decode = True
        args.workloads = "prefill-4k"
        return side_legs(args, kda, ki, hip, stream, flush, dev, {"profile_set": "prefill-4k"}, t_start)

    # ---- headline: long-1m, the largest single-GPU workload
    case = ki.make_prefill("long-1m", dev)
    res, o, fs = time_prefill(kda, case, args.steps, args.warmup, hip, stream, flush)
    rep, roof, dom = prefill_report(case, res)
    roof["traffic"] = traffic_from_profiles(dom, "long-1m")
    pipe = [traffic_from_profiles(k_, "long-1m") for k_ in ("prep", "recur")]
    roof["pipeline_traffic_ratio"] = (round(sum(pipe) / rep["alg_bytes"], 3) if all(x is not None for x in pipe)
                                      else None)
    n_chunks = (case.T_total + 63) // 64
    rep["recur_us_per_chunk_step"] = round(rep["kernel_ms_cold_median"]["recur"] * 1e3 / n_chunks, 4)
    rep["wall_ms_per_step_incl_flush"] = round(res["wall_ms"], 5)
    rep["flush_mib"] = args.flush_mib
    out = {
        "metric": METRIC, "value": round(case.T_total / (res["wall_ms"] * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["wall_ms"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16/f32",
        "data": "synthetic",
        "config": {"workload": "long-1m", "B": 1, "T": case.T_total, "H": case.H, "dk": case.dk,
                   "dv": case.dv, "chunk": 64, "inputs": "bf16", "state": "f32", "o": "f32",
                   "log_alpha": "-softplus(N(0,1)+2)", "initial_state": "N(0, 0.02)"},
        "prefill": rep,
        "roofline": roof,
    }
    # the achievable peaks of this GPU, beside the datasheet ones
    if not args.no_machine_peaks:
        mp = machine_peaks(hip, stream)
        out["machine_peaks"] = mp
        rep["mfma_frac_of_measured"] = round(rep["tflops"] / mp["bf16_mfma_tflops"], 4)
        roof["frac_of_measured_copy"] = round(roof["achieved"] / mp["copy_GBps"], 4)
    # what the oracle needs later, on the host; the GPU copies are freed
    rec_pos = None
    host = None
    if not args.no_cpu_baseline:
        g = np.random.default_rng(2024)
        rec_pos = np.unique(np.concatenate([g.integers(0, case.T_total, 4096),
                                            [0, 63, 64, 65535, 65536, case.T_total - 1]]))
        o_samp = o[torch.tensor(rec_pos, device=dev)].double().cpu().numpy()
        fs_host = fs.double().cpu().numpy()
        host = [t.cpu() for t in (case.q, case.k, case.v, case.log_alpha, case.beta, case.initial_state)]
    T_head, H_head, dk_head = case.T_total, case.H, case.dk
    del case, o, fs
    torch.cuda.empty_cache()
    if args.headline_only:
        out["env"] = environment()
        out["bench_wall_s"] = round(time.perf_counter() - t_start, 1)
        print(json.dumps(out))
        return 0

    return side_legs(args, kda, ki, hip, stream, flush, dev, out, t_start,
                     (host, rec_pos, o_samp, fs_host, T_head, H_head, dk_head) if host is not None else None)


def side_legs(args, kda, ki, hip, stream, flush, dev, out, t_start, headline_host=None):
    """Everything after the headline: the other prefill workloads, the
    comparison legs at prefill-4k size, decode-256, and the CPU baselines."""
    import numpy as np
    import torch
    # ---- the other prefill workloads, same protocol
    wls = [w for w in args.workloads.split(",") if w]
    if wls:
        out["workloads"] = {}
    case4k = None
    for wl in wls:
        c = ki.make_prefill(wl, dev)
        r_, o_, f_ = time_prefill(kda, c, max(args.steps, 20), max(args.warmup, 200 if c.T_total <= 8192 else 5),
                                  hip, stream, flush)
        wrep, wroof, wdom = prefill_report(c, r_)
        wroof["traffic"] = traffic_from_profiles(wdom, wl)
        wrep["roofline"] = wroof
        out["workloads"][wl] = wrep
        if wl == "prefill-4k":
            case4k = c
        del o_, f_
    torch.cuda.empty_cache()
    if case4k is None:
        case4k = ki.make_prefill("prefill-4k", dev)
    case = case4k
    TH = case.T_total * case.H
    if "prefill-4k" in wls:
        wall_ms = out["workloads"]["prefill-4k"]["warm_ms_median"]
    else:  # the comparisons below are against prefill-4k, warm, back to back
        r_, _, _ = time_prefill(kda, case, 20, 200, hip, stream, Flusher(0, dev))
        wall_ms = _stats(r_["warm"])[0]
    side_steps, side_warm = 20, 50  # the comparison legs (prefill-4k size, warm clocks)

    if not args.no_dplr:
        dcase = ki.make_dplr("prefill-4k", dev)
        dplr_ms, _, _ = time_dplr(kda, dcase, side_steps, side_warm)
        # per token-head, d = 128, chunk 64: four gated chunk matrices, three
        # WY/intra products, three d x d state products, output (see DESIGN)
        dplr_flops = 206165 * TH
        out["dplr_comparison"] = {
            "workload": "prefill-4k (+ a = beta a_hat, b = a_hat)", "ms_per_step": round(dplr_ms, 5),
            "tokens_per_s": round(case.T_total / (dplr_ms * 1e-3), 1),
            "tflops": round(dplr_flops / (dplr_ms * 1e-3) / 1e12, 2),
            "time_ratio_dplr_over_kda": round(dplr_ms / wall_ms, 3),
            "hbm_bytes_per_launch": {"prep": traffic_from_profiles("dplr_prep"),
                                     "recur": traffic_from_profiles("dplr_recur")}}
        del dcase

    if not args.no_bwd:
        # the backward on prefill-4k (with the per-kernel traffic), varlen-16 and
        # the 1M-token sequence (in pieces); each against its forward's time
        out["backward"] = {}
        legs = [("prefill-4k", case, 5, 3, wall_ms, "warm median")]
        if args.profile_set is None:
            wv = out.get("workloads", {}).get("varlen-16")
            legs.append(("varlen-16", None, 5, 2, wv["warm_ms_median"] if wv else None, "warm median"))
            legs.append(("long-1m", None, 2, 1, out.get("prefill", {}).get("cold_ms_median"), "cold median"))
        for wl, c, steps, warm, fwd_ms, fwd_kind in legs:
            c = c if c is not None else ki.make_prefill(wl, dev)
            bwd_ms, ws_bytes = time_bwd(kda, c, steps, warm)
            leg = {"workload": f"{wl}, d_o ~ N(0,1), d_final_state ~ N(0, 0.01)", "steps": steps,
                   "warmup": warm, "ms_per_step": round(bwd_ms, 5),
                   "tokens_per_s": round(c.T_total / (bwd_ms * 1e-3), 1),
                   "workspace_bytes": ws_bytes, "pieces": bwd_pieces(c),
                   "time_ratio_bwd_over_fwd": round(bwd_ms / fwd_ms, 3) if fwd_ms else None,
                   "fwd_time": fwd_kind}
            if wl == "prefill-4k":
                leg["hbm_bytes_per_launch"] = {k_: traffic_from_profiles(k_) for k_ in
                                               ("bwd_fwd_prep", "bwd_fwd_recur", "bwd_prep", "bwd_recur",
                                                "bwd_local")}
            out["backward"][wl] = leg
            if c is not case:
                del c
            torch.cuda.empty_cache()

    if not args.no_layer:
        lc = ki.make_layer("prefill-4k", dev)
        lt = time_layer(kda, lc, side_steps, side_warm, hip, stream)
        # compulsory bytes per token-head: prologue reads xq, xk, xv, xa (bf16, 4 x 256) and
        # xb (2), writes q, k, v, log_alpha (4 x 256) and beta (2); epilogue reads o (fp32 512)
        # and xg (256), writes y (256)
        pro_b, epi_b = 2052 * TH, 1024 * TH
        out["layer"] = {
            "workload": "prefill-4k pre-activations (bf16)",
            "ms": {k_: round(v_, 5) for k_, v_ in lt.items()},
            "tokens_per_s": round(case.T_total / (lt["layer"] * 1e-3), 1),
            "fused_tokens_per_s": round(case.T_total / (lt["fused_layer"] * 1e-3), 1),
            "one_call_tokens_per_s": round(case.T_total / (lt["one_call_layer"] * 1e-3), 1),
            "fused_prep_hbm_bytes_per_launch": traffic_from_profiles("layer_prep"),
            "one_call_recur_hbm_bytes_per_launch": traffic_from_profiles("layer_recur"),
            "prologue_roofline": {"bound": "hbm", "achieved": round(pro_b / (lt["prologue"] * 1e-3) / 1e9, 1),
                                  "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                                  "frac": round(pro_b / (lt["prologue"] * 1e-3) / PEAK_HBM, 4),
                                  "traffic": traffic_from_profiles("layer_prologue")},
            "epilogue_roofline": {"bound": "hbm", "achieved": round(epi_b / (lt["epilogue"] * 1e-3) / 1e9, 1),
                                  "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                                  "frac": round(epi_b / (lt["epilogue"] * 1e-3) / PEAK_HBM, 4),
                                  "traffic": traffic_from_profiles("layer_epilogue")}}
        del lc
        if not args.no_layer_decode:
            ld_ms, ldf_ms = time_layer_decode(kda, ki, 200, 50, hip, stream)
            out["layer"]["decode_step"] = {
                "workload": "decode-256 pre-activations (bf16), 256 sequences x 32 heads, fp32 states",
                "ms_per_step": round(ld_ms, 5), "tokens_per_s": round(256 / (ld_ms * 1e-3), 1),
                "fused_epilogue_ms_per_step": round(ldf_ms, 5),
                "fused_epilogue_tokens_per_s": round(256 / (ldf_ms * 1e-3), 1)}

    if not args.no_decode:
        dec_inputs = min(args.decode_steps, 100)  # distinct per-step inputs, cycled
        dec = ki.make_decode(256, 32, 128, dec_inputs, dev)
        dms = time_decode(kda, dec, args.decode_steps, 50, hip, stream)
        NH = 256 * 32
        state_bytes = 2 * NH * 128 * 128 * 4
        alg = state_bytes + NH * (4 * 128 * 2 + 2 + 128 * 4)
        copy_gbps = copy_bandwidth(hip, stream)
        out["decode"] = {"workload": "decode-256", "steps": args.decode_steps,
                         "ms_per_step": round(dms, 5), "state_GBps": round(state_bytes / dms / 1e6, 1),
                         "alg_GBps": round(alg / dms / 1e6, 1),
                         "hbm_frac": round(alg / dms / 1e6 / (PEAK_HBM / 1e9), 4),
                         "measured_copy_GBps": round(copy_gbps, 1),
                         "frac_of_measured_copy": round(alg / dms / 1e6 / copy_gbps, 4),
                         "roofline": {"kernel": "decode_kernel", "bound": "hbm",
                                      "achieved": round(alg / dms / 1e6, 1), "peak": PEAK_HBM / 1e9,
                                      "unit": "GB/s", "frac": round(alg / dms / 1e6 / (PEAK_HBM / 1e9), 4),
                                      "traffic": traffic_from_profiles("decode", "decode-256")}}
        del dec

    if not args.no_cpu_baseline and headline_host is not None:
        host, rec_pos, o_samp, fs_host, T_head, H_head, dk_head = headline_host
        del case
        torch.cuda.empty_cache()
        threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count() or 1
        cb, S_ref, o_rec = cpu_baseline(host, T_head, H_head, dk_head, rec_pos, threads)
        out["cpu_baseline"] = cb
        out["cpu_single_thread"] = cpu_single_thread(ki.make_prefill("prefill-4k", dev))
        # parity of this very run's headline call against the oracle's results
        rms = lambda x: float(np.sqrt(np.mean(x * x)))
        out["parity_long_1m"] = {
            "err_o_sampled": float(np.max(np.abs(o_samp - o_rec)) / rms(o_rec)),
            "err_final_state": float(np.max(np.abs(fs_host - S_ref)) / rms(S_ref)),
            "positions": int(len(rec_pos)), "heads": H_head, "tol": 2e-2}
    out["env"] = environment()
    out["bench_wall_s"] = round(time.perf_counter() - t_start, 1)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
