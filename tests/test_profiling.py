"""Host-side tests of the rocprofv3 summaries (no GPU).

The HBM traffic the benchmark reports comes from two counter runs: every
dispatch's FETCH_SIZE and WRITE_SIZE (KiB), scaled by what the same counter
reads for a device copy of known size in the same run.  These tests build
small counter files by hand and check that arithmetic, the per-launch
average over a kernel's dispatches, the match on kernel names, and that a
figure taken on other kernel sources is not reported.
"""
import csv
import json
import os

import pytest

from heterogeneous_adapter_batching_amd import profiling

COPY = "void at::native::copyBuffer<unsigned char>(unsigned char*)"
SHRINK = "void lora::(anonymous namespace)::k_shrink<unsigned short, 1, 1>(lora::ShrinkArgs)"
EXPAND = "void lora::(anonymous namespace)::k_expand_decode<unsigned short, false, 2>(lora::ExpandArgs)"
OTHER = "void at::native::vectorized_elementwise_kernel<8>(int)"


def _counters(path, counter, rows):
    """rows: (dispatch id, kernel name, value); a dispatch may span several
    rows (per-XCD instances), which are summed."""
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        for d, name, v in rows:
            w.writerow([d, name, 1024, counter, v])


@pytest.fixture()
def runs(tmp_path):
    # the copy moves 256 MiB: FETCH reads half of it (factor 2), WRITE all (factor 1)
    fetch = [(1, COPY, 131072.0), (2, SHRINK, 100.0), (2, SHRINK, 50.0), (3, SHRINK, 250.0),
             (4, EXPAND, 1000.0), (5, OTHER, 7.0)]
    write = [(1, COPY, 262144.0), (2, SHRINK, 10.0), (3, SHRINK, 30.0), (4, EXPAND, 400.0),
             (5, OTHER, 3.0)]
    fp, wp = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _counters(fp, "FETCH_SIZE", fetch)
    _counters(wp, "WRITE_SIZE", write)
    return str(fp), str(wp)


def test_short_name():
    assert profiling.short_name(SHRINK) == "k_shrink<unsigned short, 1, 1>"
    assert profiling.short_name(EXPAND).split("<")[0] == "k_expand_decode"


def test_traffic_scaling(runs):
    fp, wp = runs
    r = profiling.traffic(fp, wp, "k_shrink", 256 << 20)
    assert r["fetch"]["factor"] == pytest.approx(2.0)
    assert r["write"]["factor"] == pytest.approx(1.0)
    # dispatch 2 sums its two rows (150 KiB), dispatch 3 reads 250: 200 KiB a launch
    assert r["fetch"]["kib_per_launch"] == pytest.approx(200.0)
    assert r["fetch"]["bytes_per_launch"] == pytest.approx(200.0 * 1024 * 2)
    assert r["write"]["bytes_per_launch"] == pytest.approx(20.0 * 1024)
    assert r["fetch"]["dispatches"] == 2
    # kernels launched together add their per-launch figures
    both = profiling.traffic(fp, wp, "k_shrink+k_expand_decode", 256 << 20)
    assert both["fetch"]["kib_per_launch"] == pytest.approx(1200.0)


def test_traffic_missing_kernel(runs):
    fp, wp = runs
    with pytest.raises(SystemExit):
        profiling.traffic(fp, wp, "k_expand", 256 << 20)   # k_expand_decode is another kernel


def test_traffic_file_and_source_hash(runs, tmp_path, monkeypatch):
    import bench
    fp, wp = runs
    js, out = tmp_path / "traffic.json", tmp_path / "traffic.txt"
    profiling.main(["traffic", "--fetch", fp, "--write", wp, "--workload", "wl",
                    "--kernel", "k_expand_decode", "--copy-bytes", str(256 << 20),
                    "--json", str(js), "--out", str(out), "--command", "cmd a",
                    "--command", "cmd b"])
    ent = json.load(open(js))["wl"]["k_expand_decode"]
    assert ent["bytes_per_launch"] == pytest.approx((1000.0 * 2 + 400.0) * 1024)
    assert ent["source_hash"] == profiling.source_hash()
    text = open(out).read()
    assert "command: cmd a" in text and "command: cmd b" in text
    # the benchmark reads the figure only while the kernel sources are unchanged
    os.makedirs(tmp_path / "profiles")
    os.replace(js, tmp_path / "profiles" / "hbm_traffic.json")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profile("k_expand_decode", "wl") == pytest.approx(
        ent["bytes_per_launch"])
    monkeypatch.setattr(profiling, "source_hash", lambda: "another")
    assert bench.traffic_from_profile("k_expand_decode", "wl") is None
    assert bench.traffic_from_profile("k_shrink", "wl") is None


def test_mfma_use_per_launch_shape(tmp_path):
    """MFMA use groups dispatches by (kernel, workgroups): the busy ratio is
    averaged over a dispatch's rows, the FLOP summed, and the rate uses the
    kernel trace's average duration for that same shape."""
    cpath = tmp_path / "c.csv"
    with open(cpath, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size",
                    "Counter_Name", "Counter_Value"])
        # two dispatches of the shrink on 64 workgroups, one on 128
        for d, grid, util, fl in ((1, 64 * 256, 10.0, 2e9), (2, 64 * 256, 20.0, 4e9),
                                  (3, 128 * 256, 5.0, 1e9)):
            w.writerow([d, SHRINK, grid, 256, "MfmaUtil", util])
            w.writerow([d, SHRINK, grid, 256, "MfmaFlopsBF16", fl / 2])
            w.writerow([d, SHRINK, grid, 256, "MfmaFlopsBF16", fl / 2])
        w.writerow([4, OTHER, 256, 256, "MfmaUtil", 99.0])
    tpath = tmp_path / "t.csv"
    with open(tpath, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp",
                    "Workgroup_Size_X", "Grid_Size_X"])
        w.writerow([SHRINK, 0, 10_000, 256, 64 * 256])
        w.writerow([SHRINK, 0, 20_000, 256, 64 * 256])
        w.writerow([SHRINK, 0, 4_000, 256, 128 * 256])
    res = profiling.mfma_use(str(cpath), str(tpath), ["k_shrink"])
    assert set(res) == {("k_shrink", 64), ("k_shrink", 128)}
    a = res[("k_shrink", 64)]
    assert a["util"] == pytest.approx(15.0)
    assert a["gflop"] == pytest.approx(3.0)
    assert a["us"] == pytest.approx(15.0)
    assert a["launches"] == 2
    txt = profiling.mfma_summary(str(cpath), str(tpath), ["k_shrink"], ["cmd"])
    # 3 GFLOP in 15 us = 200 TFLOP/s = 0.08 of the bf16 peak
    assert "200.00" in txt and "0.0800" in txt


def test_copy_overlap_split(tmp_path):
    """A launch is "with a copy" when any copy interval overlaps it, also a
    copy that began long before it; touching endpoints do not count."""
    t = tmp_path / "t.csv"
    with open(t, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp",
                    "Workgroup_Size_X", "Grid_Size_X"])
        for s0, s1 in ((0, 1000), (1000, 3000), (5000, 6000), (9000, 9500), (20000, 22000)):
            w.writerow([EXPAND, s0, s1, 256, 64 * 256])
        w.writerow([OTHER, 5000, 6000, 256, 256])
    c = tmp_path / "c.csv"
    with open(c, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kind", "Start_Timestamp", "End_Timestamp"])
        w.writerow(["MEMORY_COPY", 3000, 5500])     # overlaps the third, touches the second
        w.writerow(["MEMORY_COPY", 8000, 30000])    # covers the fourth and fifth
    res = profiling.copy_overlap(str(t), str(c), ["k_expand_decode"])
    alone, na, with_copy, nb = res[("k_expand_decode", 64)]
    assert (na, nb) == (2, 3)
    assert alone == pytest.approx((1.0 + 2.0) / 2)
    assert with_copy == pytest.approx((1.0 + 0.5 + 2.0) / 3)
