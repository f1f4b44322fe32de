"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer: the
C-ABI library's argument checks, layout and split arithmetic (kvq_api.cpp,
kvq_plan.cpp; the kernels are not instrumented) and the C oracle, driven by
the ABI, oracle and quantizer tests in a child process with the clang ASan
runtime preloaded.  Any report fails the run (halt on the first one)."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FILES = ["tests/test_abi.py", "tests/test_oracle.py", "tests/test_oracle_prefill.py", "tests/test_quant_fastpath.py"]


def test_host_code_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from decode_attention_asym_amd import build
    import oracle
    lib = build.build_sanitized()
    runtime = build.san_runtime()
    clang = os.path.join(os.path.dirname(build.HIPCC), "..", "lib", "llvm", "bin", "clang")
    olib = oracle.build_sanitized(os.path.normpath(clang))
    logs = str(tmp_path / "san")
    env = dict(os.environ,
               LD_PRELOAD=runtime,
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=1:detect_odr_violation=0:alloc_dealloc_mismatch=0:log_path={logs}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={logs}",
               KVQ_LIB=lib, KVQ_ORACLE_LIB=olib)
    r = subprocess.run([sys.executable, "-m", "pytest", *FILES, "-q", "-m", "not gpu", "-x", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    reports = "".join(open(f).read() for f in glob.glob(logs + "*"))
    assert r.returncode == 0 and not reports, (r.stdout[-3000:], r.stderr[-3000:], reports[:4000])
    assert " passed" in r.stdout, r.stdout[-2000:]
