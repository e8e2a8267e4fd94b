"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The C-ABI library (argument checks, workspace sizing, plans: la_api.cpp and
the host side of every launcher) is rebuilt with host sanitizers and the
oracle (la_oracle.c) likewise; the ABI tests and the oracle's pins then run
in a child process that preloads the shared ASan runtime and loads those
builds (LA_LIBRARY, LAO_LIBRARY).  Any invalid access, overflow or undefined
operation aborts the child and fails this test.  No GPU is used: the ABI
tests call with fake device pointers that the checks reject before any HIP
call."""
import os
import shutil
import subprocess
import sys

import pytest

from linear_attention_phi_amd import build as labuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_and_oracle_under_host_sanitizers(tmp_path):
    if not shutil.which(labuild._hipcc()) and not os.path.exists(labuild._hipcc()):
        pytest.skip("hipcc is not installed")
    runtime = labuild.asan_runtime()
    if runtime is None:
        pytest.skip("the compiler's shared ASan runtime is not installed")
    import oracle

    lib = labuild.build_sanitized()
    olib = oracle.build_sanitized(str(tmp_path / "liblaoracle_san.so"))
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, LA_LIBRARY=lib, LAO_LIBRARY=olib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_oracle.py")]
    res = subprocess.run(cmd, cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    print(tail)
    assert res.returncode == 0, f"sanitized run failed ({res.returncode}):\n{tail}"
    assert " passed" in res.stdout
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr
