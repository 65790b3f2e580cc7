"""The host-side code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the C oracle and the library's host code (argument validation,
workspace planning, the binding's calls through the C ABI) are rebuilt with
both sanitizers, and the oracle pins, the ABI host tests and the binding host
tests run against those builds in a child process with the sanitizer runtime
preloaded. Any sanitizer report fails the test. Device code is built as usual
(no GPU sanitizer is used); nothing here touches a GPU."""
import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/llvm"
RUNTIMES = sorted(glob.glob(os.path.join(LLVM, "lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")))
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not RUNTIMES or not os.path.exists(os.path.join(LLVM, "bin/clang")),
                    reason="the ROCm clang sanitizer runtime is not installed")
def test_host_code_clean_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from gated_delta_rule_41_amd import build as hip_build
    with tempfile.TemporaryDirectory() as tmp:
        oracle_so = os.path.join(tmp, "liboracle_san.so")
        subprocess.run([os.path.join(LLVM, "bin/clang"), "-O1", "-g", *SAN, "-shared-libasan", "-fopenmp",
                        "-fPIC", "-shared", "-std=c11", os.path.join(ROOT, "oracle", "kda_oracle.c"),
                        "-o", oracle_so, "-lm"], check=True)
        host_only = [x for f in SAN for x in ("-Xarch_host", f)]  # host code only
        kda_so = hip_build.build(extra=host_only, out=os.path.join(tmp, "libkda_san.so"),
                                 build_dir=os.path.join(tmp, "obj"),
                                 link_extra=["-shared-libasan", "-fsanitize=address,undefined"])
        logs = os.path.join(tmp, "report")
        env = dict(os.environ, LD_PRELOAD=RUNTIMES[-1], KDA_LIBRARY=kda_so, KDA_ORACLE_LIBRARY=oracle_so,
                   ASAN_OPTIONS=f"detect_leaks=0:log_path={logs}",
                   UBSAN_OPTIONS=f"print_stacktrace=1:log_path={logs}")
        res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                              os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                              os.path.join(ROOT, "tests", "test_abi_host.py"),
                              os.path.join(ROOT, "tests", "test_binding_host.py")],
                             cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        reports = [open(f).read() for f in glob.glob(logs + ".*")]
        assert not reports, "\n".join(r[:4000] for r in reports)
        assert res.returncode == 0, res.stdout[-4000:]
