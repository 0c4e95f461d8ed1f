"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the host library (pool, plan, validation, exchange bookkeeping; no
device code) and the CPU oracle with -fsanitize=address,undefined, then runs
the host-side library tests and the oracle's pin tests against those builds
in a child process (the sanitizer runtime must be loaded first).  Any report
ends the child with an error.  No GPU is used.
"""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
from heterogeneous_adapter_batching_amd import build as lib_build  # noqa: E402
from oracle import build as oracle_build  # noqa: E402


def _runtime(name):
    out = subprocess.run(["g++", f"-print-file-name={name}"], stdout=subprocess.PIPE,
                         text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_host_code_under_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no libasan for g++")
    lib = lib_build.host_sanitized(str(tmp_path / "libhab_lora_san.so"))
    orc = oracle_build.build(str(tmp_path / "liboracle_san.so"),
                             extra=["-g", "-O1", *lib_build.SANITIZE])
    env = dict(os.environ, HAB_LORA_LIB=lib, HAB_ORACLE_LIB=orc, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu and not slow",
                          "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_library.py"),
                          os.path.join(ROOT, "tests", "test_oracle.py")],
                         cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                         text=True, timeout=900)
    tail = "\n".join(res.stdout.splitlines()[-40:])
    assert res.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in res.stdout and "runtime error:" not in res.stdout, tail
    assert " passed" in tail, tail
