"""The benchmark's contract and its byte accounting (CPU only)."""
import os
import subprocess
import sys

import numpy as np

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402
from synth import config  # noqa: E402


def test_more_than_one_gpu_refused():
    """--gpus 2 exits with status 2 and says why, before touching a GPU."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_full_stack_algorithmic_bytes():
    """The full stack's algorithmic bytes, counted independently: each
    distinct adapter's 32 layers x 7 projections at rank 16 (83,886,080 B in
    bf16), each of the 4 activations once per layer, base_out read and y
    written once per projection."""
    w = config(4)
    alg = bench.algorithmic(w)
    distinct = len({int(a) for a in w.seg_adapter if a >= 0})
    per_adapter = 32 * 16 * sum(p.h_in + p.h_out for p in w.projs) * 2
    assert per_adapter == 83_886_080
    x = 32 * 128 * (4096 + 4096 + 4096 + 14336) * 2
    y = 32 * 128 * sum(p.h_out for p in w.projs) * 2 * 2
    assert alg["adapter"] == distinct * per_adapter
    assert alg["bytes"] == distinct * per_adapter + x + y
    flops = 32 * 128 * sum(2 * 16 * (p.h_in + p.h_out) for p in w.projs)
    assert alg["flops"] == flops


def test_kernel_bytes_sum_to_the_step():
    """Per-launch bytes of the shrink and expand over one layer's calls add up
    to the step's algorithmic bytes per layer plus the float32 v the two
    kernels hand over (written once, read once)."""
    w = config(4)
    alg = bench.algorithmic(w)
    per_layer = sum(bench.kernel_bytes(w, c, k) for c in w.calls for k in ("shrink", "expand"))
    tok = w.token_adapter()
    v = sum(4 * int(w.ranks[tok[t]]) * len(c) for c in w.calls for t in range(w.num_tokens)
            if tok[t] >= 0)
    assert np.isclose(per_layer, alg["bytes"] / w.num_layers + 2 * v)
