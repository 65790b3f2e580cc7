"""Benchmark of the KDA hot path on one MI355X.

One step = one chunkwise prefill call (per-chunk preparation, then the
inter-chunk state recursion with the chunk outputs fused in) on the
``prefill-4k`` workload: B=1, H=32,
T=4096, dk=dv=128, chunk 64, bf16 inputs, fp32 initial/final state and fp32
output (synthetic, seeded; see kda_inputs). The decode step (the remaining row
of the hot path) is timed in the same run on ``decode-256`` (256 sequences x 32
heads, fp32 states of 512 MiB, updated in place) and reported in the same JSON
line. Prints ONE JSON line. The general-DPLR comparison operator (the transition KDA specialises,
with free low-rank vectors a, b) is timed on the same workload and reported
beside it under "dplr_comparison", the chunkwise backward (gradients of
q, k, v, log_alpha, beta and the initial state) under "backward", and the layer
around the operator (prologue, operator, epilogue) under "layer".

    python bench.py [--steps K] [--warmup W] [--decode-steps S] [--no-cpu-baseline] [--no-dplr]
                    [--no-bwd] [--no-layer]

Profiling helpers (used to write the summaries under profiles/):
    python bench.py --copy-calibration MIB        # counter calibration kernel only
    python bench.py --report-trace DB             # kernel-trace database -> markdown
    python bench.py --report-pmc FETCH_DB WRITE_DB CAL_FETCH_DB CAL_WRITE_DB CAL_BYTES
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
KERNEL_BYTES_PER_TOKEN_HEAD = {            # compulsory traffic of each prefill kernel
    "prep": 1026 + 1160,                   # reads q,k,v,log_alpha,beta; writes Q+,K-,W,U,A_qk,gamma
    # with bf16 inputs the output is fused into the state recursion:
    "recur": 776 + 384 + 512,              # reads W,K-,U,gamma,Q+,A_qk; writes o (fp32)
}
# fp32 inputs (not benchmarked) run the unfused pair: recursion 776 + 768 (h_n,
# V_new written), output 1152 + 512
KERNEL_SYMBOL = {"prep": "prep_kernel", "recur": "recur_kernel", "decode": "decode_kernel",
                 "dplr_prep": "dplr_prep_kernel", "dplr_recur": "recur_kernel",
                 "bwd_fwd_prep": "prep_kernel", "bwd_fwd_recur": "recur_kernel",
                 "bwd_prep": "bwd_prep_kernel", "bwd_recur": "recur_kernel", "bwd_local": "bwd_local_kernel",
                 "layer_prologue": "layer_prologue_kernel", "layer_epilogue": "layer_epilogue_kernel",
                 "layer_prep": "prep_kernel"}
KERNEL_SOURCE = {"prep": "kda_prep.hip", "recur": "kda_recur.hip", "decode": "kda_decode.hip",
                 "dplr_prep": "kda_dplr_prep.hip", "dplr_recur": "kda_recur.hip",
                 "bwd_fwd_prep": "kda_prep.hip", "bwd_fwd_recur": "kda_recur.hip",
                 "bwd_prep": "kda_bwd.hip", "bwd_recur": "kda_recur.hip", "bwd_local": "kda_bwd.hip",
                 "layer_prologue": ("kda_layer.hip", "kda_layer_util.h"), "layer_epilogue": "kda_layer.hip",
                 "layer_prep": ("kda_prep.hip", "kda_layer_util.h")}


def kernel_key(short_name: str):
    """Which of this library's kernels a demangled name (arguments stripped) is.
    The template arguments tell the instantiations apart: the preparation's
    last two are fp32 factors (the backward's forward recompute) and the fused
    layer prologue; the state
    recursion's are <D, fp32 factors, fused output, fp32 output, DPLR chain,
    added per-chunk term (the backward's state-gradient recursion)>."""
    if "<" not in short_name:
        return None
    sym, args = short_name.split("<", 1)
    args = [x.strip() for x in args.rstrip(">").split(",")]
    flag = lambda i: len(args) > i and args[i] == "true"
    if sym == "recur_kernel":
        if flag(5):
            return "bwd_recur"
        if flag(4):
            return "dplr_recur"
        return "bwd_fwd_recur" if flag(1) else "recur"
    if sym == "prep_kernel":  # <D, TIn, TG, fp32 factors, fused layer prologue>
        if flag(4):
            return "layer_prep"
        return "bwd_fwd_prep" if flag(3) else "prep"
    for key in ("dplr_prep", "decode", "bwd_prep", "bwd_local", "layer_prologue", "layer_epilogue"):
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


def traffic_from_profiles(kernel: str, units: int):
    """HBM bytes per launch from committed rocprofv3 --pmc counters, if they were
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel}_prefill-4k.json" if kernel != "decode"
                        else "pmc_decode_decode-256.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha") != source_sha(kernel):
        return None
    return rec.get("bytes_per_launch")


def time_prefill(kda, case, steps, warmup, hip, stream):
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
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    # per-kernel durations: HIP events at the stage boundaries, on the launch stream
    ev = Events(hip, 4 * steps)
    for s in range(steps):
        call(events=ev.ev[4 * s:4 * s + 4])
    torch.cuda.synchronize()
    per = {"prep": 0.0, "recur": 0.0}
    span = 0.0
    for s in range(steps):
        b = 4 * s
        per["prep"] += ev.ms(b, b + 1)
        per["recur"] += ev.ms(b + 1, b + 3)  # state recursion with the fused output
        span += ev.ms(b, b + 3)
    ev.close()
    per = {k_: v_ / steps for k_, v_ in per.items()}
    return wall_ms, per, span / steps, o, fs


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


def time_bwd(kda, case, steps, warmup):
    """Whole-call time of the chunkwise backward (its five kernels: the fp32
    forward recompute, the operand preparation, the reverse state-gradient
    recursion and the local adjoints), torch events on torch's current stream,
    which the binding launches on."""
    import torch
    dev = case.q.device
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    d_o = torch.randn(case.T_total, case.H, case.dv, generator=g, device=dev)
    d_fin = torch.randn(case.N, case.H, case.dk, case.dv, generator=g, device=dev) * 0.1
    ws = torch.empty(kda.bwd_workspace_size(case.N, case.T_total, case.H, case.dk, case.dv),
                     dtype=torch.uint8, device=dev)

    def call():
        return kda.chunk_bwd(case.q, case.k, case.v, case.log_alpha, case.beta, d_o, case.initial_state,
                             case.cu_seqlens, d_fin, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g_ = call()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, g_, ws.numel()


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
    return out


def time_layer_decode(kda, ki, steps, warmup, hip, stream, N=256, H=32, d=128):
    """The layer's decode step at decode-256 size (one bf16 token per sequence):
    decode prologue (history in place), kda_decode_step (fp32 state in place),
    epilogue, all through the C ABI between two events around the loop.
    Returns ms per step."""
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

    def step():
        if lib.kda_layer_decode_prologue(*pro) != 0 or lib.kda_decode_step(*dec) != 0 or \
                lib.kda_layer_epilogue(*epi) != 0:
            raise RuntimeError("layer decode step failed")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = Events(hip, 2)
    ev.record(0, stream)
    for _ in range(steps):
        step()
    ev.record(1, stream)
    torch.cuda.synchronize()
    ms = ev.ms(0, 1) / steps
    ev.close()
    return ms


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


def cpu_baseline(case):
    """The oracle (fp64 token recurrence, OpenMP over (sequence, head, column
    block)) on the host cores, on the same prefill-4k inputs copied to host."""
    import oracle
    host = [t.cpu() for t in (case.q, case.k, case.v, case.log_alpha, case.beta, case.initial_state)]
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count() or 1
    heads = list(range(case.H))
    reps, t0 = 0, time.perf_counter()
    while True:  # whole passes over the workload until about 10 s of host work
        oracle.recurrence(*host, None, heads=heads, want_o=True, col_blocks=2, threads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or reps >= 1000:
            break
    return {"value": reps * case.T_total / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"prefill-4k in full (T={case.T_total}, H={case.H}, d={case.dk}, fp64 token "
                      f"recurrence), {reps} passes in {dt:.1f} s wall"}, host


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


def report_pmc(fetch_db: str, write_db: str, cal_fetch_db: str, cal_write_db: str, cal_bytes: int) -> int:
    """HBM traffic per launch of each library kernel from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch, one rocprofv3 --pmc run each), each scaled by
    what the same counter reads for the calibration copy kernel of known size.
    Writes profiles/pmc_<kernel>_<workload>.json (read back by the roofline
    report while the kernel source is unchanged) and prints a markdown table."""
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
        wl = "decode-256" if kern == "decode" else "prefill-4k"
        rec = {"kernel": name, "workload": wl, "source_sha": source_sha(kern),
               "fetch_kib": fe[name][1], "write_kib": wr[name][1],
               "fetch_scale": f_fetch, "write_scale": f_write, "bytes_per_launch": round(b)}
        with open(os.path.join(ROOT, "profiles", f"pmc_{kern}_{wl}.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
    return 0


def main(argv=None):
    if argv is None:
        argv = sys.argv[1:]
    if argv[:1] == ["--report-trace"]:
        return report_trace(argv[1])
    if argv[:1] == ["--report-pmc"]:
        return report_pmc(argv[1], argv[2], argv[3], argv[4], int(argv[5]))
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed prefill steps first (500 take ~80 ms and bring the GPU to steady clocks)")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    case = ki.make_prefill("prefill-4k", dev)
    TH = case.T_total * case.H
    wall_ms, per, span_ms, o, fs = time_prefill(kda, case, args.steps, args.warmup, hip, stream)
    tokens_per_s = case.T_total / (wall_ms * 1e-3)
    flops = FLOP_PER_TOKEN_HEAD * TH
    tflops = flops / (wall_ms * 1e-3) / 1e12
    alg_bytes = ALG_BYTES_PER_TOKEN_HEAD * TH + 2 * case.N * case.H * case.dk * case.dv * 4
    ai = flops / alg_bytes
    ceiling = min(PEAK_BF16, ai * PEAK_HBM)

    dom = max(per, key=per.get)
    kb = KERNEL_BYTES_PER_TOKEN_HEAD[dom] * TH
    if dom == "recur":  # plus the initial and final states
        kb += 2 * case.N * case.H * case.dk * case.dv * 4
    achieved = kb / (per[dom] * 1e-3) / 1e9
    roof = {"kernel": KERNEL_SYMBOL[dom], "bound": "hbm", "achieved": round(achieved, 1),
            "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": round(achieved / (PEAK_HBM / 1e9), 4),
            "traffic": traffic_from_profiles(dom, TH), "avg_launch_ms": round(per[dom], 5),
            "alg_bytes_per_launch": kb}

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16/f32",
        "data": "synthetic",
        "config": {"workload": "prefill-4k", "B": 1, "T": case.T_total, "H": case.H, "dk": case.dk,
                   "dv": case.dv, "chunk": 64, "inputs": "bf16", "state": "f32", "o": "f32",
                   "log_alpha": "-softplus(N(0,1)+2)"},
        "prefill": {"tflops": round(tflops, 2), "mfma_peak_frac": round(tflops * 1e12 / PEAK_BF16, 4),
                    "alg_roofline_frac": round(flops / (wall_ms * 1e-3) / ceiling, 4),
                    "alg_ceiling_tflops": round(ceiling / 1e12, 1),
                    "kernel_ms": {k_: round(v_, 5) for k_, v_ in per.items()},
                    "event_span_ms": round(span_ms, 5)},
        "roofline": roof,
    }

    if not args.no_dplr:
        dcase = ki.make_dplr("prefill-4k", dev)
        dplr_ms, _, _ = time_dplr(kda, dcase, args.steps, max(3, min(200, args.warmup)))
        # per token-head, d = 128, chunk 64: four gated chunk matrices, three
        # WY/intra products, three d x d state products, output (see DESIGN)
        dplr_flops = 206165 * TH
        out["dplr_comparison"] = {
            "workload": "prefill-4k (+ a = beta a_hat, b = a_hat)", "ms_per_step": round(dplr_ms, 5),
            "tokens_per_s": round(case.T_total / (dplr_ms * 1e-3), 1),
            "tflops": round(dplr_flops / (dplr_ms * 1e-3) / 1e12, 2),
            "time_ratio_dplr_over_kda": round(dplr_ms / wall_ms, 3),
            "hbm_bytes_per_launch": {"prep": traffic_from_profiles("dplr_prep", TH),
                                     "recur": traffic_from_profiles("dplr_recur", TH)}}
        del dcase

    if not args.no_bwd:
        bwd_ms, _, ws_bytes = time_bwd(kda, case, max(5, args.steps // 5), max(3, min(50, args.warmup)))
        out["backward"] = {
            "workload": "prefill-4k, d_o ~ N(0,1), d_final_state ~ N(0, 0.01)",
            "ms_per_step": round(bwd_ms, 5), "tokens_per_s": round(case.T_total / (bwd_ms * 1e-3), 1),
            "time_ratio_bwd_over_fwd": round(bwd_ms / wall_ms, 3), "workspace_bytes": ws_bytes,
            "hbm_bytes_per_launch": {k_: traffic_from_profiles(k_, TH) for k_ in
                                     ("bwd_fwd_prep", "bwd_fwd_recur", "bwd_prep", "bwd_recur", "bwd_local")}}

    if not args.no_layer:
        lc = ki.make_layer("prefill-4k", dev)
        lt = time_layer(kda, lc, max(10, args.steps // 5), max(3, min(50, args.warmup)), hip, stream)
        # compulsory bytes per token-head: prologue reads xq, xk, xv, xa (bf16, 4 x 256) and
        # xb (2), writes q, k, v, log_alpha (4 x 256) and beta (2); epilogue reads o (fp32 512)
        # and xg (256), writes y (256)
        pro_b, epi_b = 2052 * TH, 1024 * TH
        out["layer"] = {
            "workload": "prefill-4k pre-activations (bf16)",
            "ms": {k_: round(v_, 5) for k_, v_ in lt.items()},
            "tokens_per_s": round(case.T_total / (lt["layer"] * 1e-3), 1),
            "fused_tokens_per_s": round(case.T_total / (lt["fused_layer"] * 1e-3), 1),
            "fused_prep_hbm_bytes_per_launch": traffic_from_profiles("layer_prep", TH),
            "prologue_roofline": {"bound": "hbm", "achieved": round(pro_b / (lt["prologue"] * 1e-3) / 1e9, 1),
                                  "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                                  "frac": round(pro_b / (lt["prologue"] * 1e-3) / PEAK_HBM, 4),
                                  "traffic": traffic_from_profiles("layer_prologue", TH)},
            "epilogue_roofline": {"bound": "hbm", "achieved": round(epi_b / (lt["epilogue"] * 1e-3) / 1e9, 1),
                                  "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                                  "frac": round(epi_b / (lt["epilogue"] * 1e-3) / PEAK_HBM, 4),
                                  "traffic": traffic_from_profiles("layer_epilogue", TH)}}
        del lc
        if not args.no_layer_decode:
            ld_ms = time_layer_decode(kda, ki, 200, 50, hip, stream)
            out["layer"]["decode_step"] = {
                "workload": "decode-256 pre-activations (bf16), 256 sequences x 32 heads, fp32 states",
                "ms_per_step": round(ld_ms, 5), "tokens_per_s": round(256 / (ld_ms * 1e-3), 1)}

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
                                      "traffic": traffic_from_profiles("decode", NH)}}
        del dec

    if not args.no_cpu_baseline:
        import numpy as np
        cb, host = cpu_baseline(case)
        out["cpu_baseline"] = cb
        # spot parity of this very run against the oracle (head 0, all tokens)
        import oracle
        o_ref, s_ref, _ = oracle.recurrence(*host, None, heads=[0], col_blocks=8)
        oo = o[:, 0].double().cpu().numpy()
        ss = fs[0, 0].double().cpu().numpy()
        e_o = float(np.max(np.abs(oo - o_ref[:, 0])) / np.sqrt(np.mean(o_ref[:, 0] ** 2)))
        e_s = float(np.max(np.abs(ss - s_ref[0, 0])) / np.sqrt(np.mean(s_ref[0, 0] ** 2)))
        out["parity_head0"] = {"err_o": e_o, "err_state": e_s, "tol": 2e-2}
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
