"""The library driven from C through its ABI alone (tests/c_abi/sgmv_from_c.c):
pool, plan, workspace and the sgmv calls with HIP runtime memory and a HIP
stream, against the C oracle; the two-step calls give the fused call's bits
and a refused call enqueues nothing."""
import os
import subprocess

import pytest

from conftest import ROOT

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

BIN = os.path.join(ROOT, "tests", "c_abi", "sgmv_from_c")


def test_c_program():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(BIN), "build it first (__graft_entry__.build())"
    print("[c-abi] tests/c_abi/sgmv_from_c", flush=True)
    res = subprocess.run([BIN], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                         timeout=60)
    print(res.stdout, flush=True)
    assert res.returncode == 0, res.stdout
    assert "C ABI: all checks passed" in res.stdout
