"""Build the HIP library ``libkda.so`` (gfx950 only) in-tree with hipcc.

Every source under ``csrc/`` is compiled to its own object (in parallel),
then linked into ``gated_delta_rule_41_amd/libkda.so``. Packed-fp32 VALU
instructions are disabled for the device code; hipcc's host pass warns that it
does not know that target feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkda.so")
# the benchmark's machine probes (achievable MFMA and copy rates), a library of their own
PROBE_SRC = os.path.join(PKG, "probe", "kda_probe.hip")
PROBE_LIB = os.path.join(PKG, "libkda_probe.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libkda.so)")


# per-source device-compiler options
FILE_FLAGS = {
    # keep the recurrence's MFMA accumulators (the state) in VGPRs: the state is
    # converted to fp16 operands every chunk, and AGPR<->VGPR moves would sit on
    # the sequential chain
    "kda_recur.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    # the MFMA probe's accumulators likewise (as AGPRs they are shuffled between
    # loop iterations with moves that sit between the products)
    "kda_probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, extra, build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc()] + HIPCC_FLAGS + FILE_FLAGS.get(os.path.basename(src), []) + list(extra) + ["-c", src, "-o", obj]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in res.stdout.splitlines() if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(extra=(), jobs: int = 8, verbose: bool = False, out: str = LIB, build_dir: str = BUILD,
          link_extra=()) -> str:
    """Compile every csrc/*.hip and link libkda.so (or ``out``). Always
    recompiles. ``extra`` / ``link_extra`` add compiler / linker options (the
    host-sanitizer build of the tests uses them, with its own out and build_dir)."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, build_dir), srcs))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + list(link_extra) + ["-o", tmp] + objs
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def build_probe(verbose: bool = False) -> str:
    """Compile and link the machine probes into libkda_probe.so. Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    obj = _compile(PROBE_SRC, ())
    tmp = PROBE_LIB + ".tmp"
    res = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, obj],
                         stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}")
    return PROBE_LIB


if __name__ == "__main__":
    build(verbose=True)
    build_probe(verbose=True)
