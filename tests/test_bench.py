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


def test_merge_stack_algorithmic_bytes():
    """The merged full stack (2 adapters a request): adapter bytes over the
    distinct adapters of both slots, activations once (every token has an
    adapter), y read and written once, FLOPs for both slots of every token;
    the two slots of a request name different adapters."""
    from synth import merge_full_stack
    w = merge_full_stack(2)
    assert w.merge_ids.shape == (128, 2) and (w.merge_ids[:, 0] != w.merge_ids[:, 1]).all()
    assert (w.merge_ids[:, 0] == config(4).seg_adapter).all()
    assert ((w.merge_w >= 0.2) & (w.merge_w < 1.0)).all()
    alg = bench.algorithmic(w)
    distinct = len({int(a) for a in w.merge_ids.ravel()})
    per_adapter = 83_886_080
    x = 32 * 128 * (4096 + 4096 + 4096 + 14336) * 2
    y = 32 * 128 * sum(p.h_out for p in w.projs) * 2 * 2
    assert alg["adapter"] == distinct * per_adapter
    assert alg["bytes"] == distinct * per_adapter + x + y
    assert alg["flops"] == 2 * 32 * 128 * sum(2 * 16 * (p.h_in + p.h_out) for p in w.projs)
    per_layer = sum(bench.kernel_bytes(w, c, k) for c in w.calls for k in ("shrink", "expand"))
    assert np.isclose(per_layer, alg["bytes"] / w.num_layers)


def test_kernel_bytes_sum_to_the_step():
    """Per-launch bytes of the shrink and expand over one layer's calls add up
    to the step's algorithmic bytes per layer exactly (the float32
    intermediate the two kernels hand over is not algorithmic)."""
    for ci in (1, 2, 3, 4):
        w = config(ci)
        alg = bench.algorithmic(w)
        per_layer = sum(bench.kernel_bytes(w, c, k) for c in w.calls
                        for k in ("shrink", "expand"))
        assert np.isclose(per_layer, alg["bytes"] / w.num_layers), ci


def test_step_metrics_fractions():
    """The derived figures of a step: tokens/s, GB/s and TFLOP/s from the
    algorithmic counts, the attainable roof min(MFMA peak, intensity x HBM
    peak), and for a decode workload the attainable fraction equals the HBM
    fraction (its roof is the bandwidth one)."""
    w = config(4)
    alg = bench.algorithmic(w)
    m = bench.step_metrics(w, 2.0)
    assert np.isclose(m["tokens_per_s"], 128 / 2e-3, rtol=1e-6)
    assert np.isclose(m["hbm_gbs"], alg["bytes"] / 2e-3 / 1e9, rtol=1e-4)
    assert np.isclose(m["attainable_frac"], m["hbm_frac"], rtol=1e-3)
    w2 = config(2)
    m2 = bench.step_metrics(w2, 0.1)
    a2 = bench.algorithmic(w2)
    assert np.isclose(m2["attainable_tflops"],
                      a2["flops"] / a2["bytes"] * bench.HBM_PEAK_GBS / 1e3, rtol=1e-3)
    assert m2["mfma_frac"] < m2["attainable_frac"]
