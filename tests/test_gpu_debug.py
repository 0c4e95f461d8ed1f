"""The bounds-checked debug build of the library on the GPU.

tests/debug_run.py runs in a process of its own with HAB_LORA_LIB naming
libhab_lora_debug.so (this process has the release build loaded): good
batches give the oracle's delta with no failed check, and plan tables
overwritten as a stray write would leave them set the matching check bits
while every launch completes.
"""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def test_debug_build_checks():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from heterogeneous_adapter_batching_amd import build
    assert os.path.exists(build.DEBUG_LIB), "build the library first (__graft_entry__.build())"
    print("[debug] tests/debug_run.py with the debug build", flush=True)
    res = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "tests", "debug_run.py")],
                         env=dict(os.environ, HAB_LORA_LIB=build.DEBUG_LIB), cwd=ROOT,
                         stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=100)
    print(res.stdout[-4000:], flush=True)
    assert res.returncode == 0, res.stdout[-4000:]
    assert "[debug] all checks passed" in res.stdout
