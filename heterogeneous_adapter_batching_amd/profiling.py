"""Summaries of rocprofv3 output for the kernels of this library.

Four jobs, all on CSV files that ``rocprofv3 --output-format csv`` writes:

* ``stats``: the per-kernel table of a ``--kernel-trace --stats`` run
  (``*_kernel_stats.csv``), reduced to a short text summary.
* ``traffic``: HBM bytes per launch of one kernel from two ``--pmc`` runs,
  one with ``FETCH_SIZE`` and one with ``WRITE_SIZE`` (both KiB per
  dispatch).  Each counter is scaled by what it reads for a plain device copy
  of known size in the same run (a copy of N bytes reads N and writes N), so
  the figure is in the copy's bytes.  The result is stored with a hash of the
  kernel sources; a reader that finds a different hash treats it as absent.
* ``mfma``: MFMA use per launch shape from a ``--pmc MfmaUtil MfmaFlopsBF16``
  run, turned into a rate with the kernel trace of the same workload.
* ``overlap``: kernel durations with and without a host-to-device copy in
  flight, from a ``--kernel-trace --memory-copy-trace`` run.

Usage::

    python -m heterogeneous_adapter_batching_amd.profiling stats CSV --command CMD --out TXT
    python -m heterogeneous_adapter_batching_amd.profiling traffic --fetch CSV --write CSV \\
        --workload NAME --kernel K --copy-bytes N --json OUT --out TXT --command CMD ...
    python -m heterogeneous_adapter_batching_amd.profiling mfma COUNTER_CSV TRACE_CSV \\
        --kernel K --command CMD --command CMD --out TXT
    python -m heterogeneous_adapter_batching_amd.profiling overlap TRACE_CSV COPY_CSV \\
        --kernel K --command CMD --out TXT
"""
from __future__ import annotations

import argparse
import bisect
import csv
import hashlib
import json
import os
import re
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_SOURCES = ("kernels.hip", "lora_sgmv.cpp", "sgmv_internal.h")
_COPY = re.compile(r"copyBuffer")


def source_hash() -> str:
    """Hash of the kernel and launcher sources the counters were taken on."""
    h = hashlib.sha256()
    for f in _SOURCES:
        with open(os.path.join(ROOT, "heterogeneous_adapter_batching_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    """Kernel name without namespaces, arguments or template arguments."""
    n = re.sub(r"lora::\(anonymous namespace\)::", "", name.replace("void ", ""))
    n = re.sub(r"\(.*", "", n)
    return n.strip()


def _rows(path):
    with open(path, newline="") as f:
        rd = csv.DictReader(f)
        for r in rd:
            yield {k.strip().lower(): v for k, v in r.items() if k}


def kernel_stats(path: str, command: str, limit: int = 12) -> str:
    rows = list(_rows(path))
    rows.sort(key=lambda r: -float(r.get("totaldurationns", 0)))
    out = ["# rocprofv3 --kernel-trace --stats", f"command: {command}", "",
           f"{'kernel':60s} {'calls':>6s} {'avg_us':>9s} {'min_us':>8s} {'max_us':>8s} {'pct':>6s}"]
    for r in rows[:limit]:
        out.append(f"{r['name'][:60]:60s} {int(r['calls']):6d} "
                   f"{float(r['averagens']) / 1e3:9.2f} {float(r['minns']) / 1e3:8.2f} "
                   f"{float(r['maxns']) / 1e3:8.2f} {float(r['percentage']):6.2f}")
    return "\n".join(out) + "\n"


def launches_by_grid(path: str, limit: int = 12) -> str:
    """Per (kernel, workgroups) durations from a ``*_kernel_trace.csv``: the
    launches of one call shape (e.g. one projection set) share a grid."""
    groups = defaultdict(list)
    for r in _rows(path):
        wg = int(r.get("workgroup_size_x") or r.get("workgroup_size") or 1)
        g = int(r.get("grid_size_x") or r.get("grid_size") or 0) // max(wg, 1)
        groups[(short_name(r["kernel_name"]), g)].append(
            (int(r["end_timestamp"]) - int(r["start_timestamp"])) / 1e3)
    total = sum(sum(v) for v in groups.values())
    out = [f"{'kernel':40s} {'wgs':>6s} {'calls':>6s} {'avg_us':>8s} {'med_us':>8s} {'pct':>6s}"]
    for (name, g), v in sorted(groups.items(), key=lambda kv: -sum(kv[1]))[:limit]:
        v = sorted(v)
        out.append(f"{name[:40]:40s} {g:6d} {len(v):6d} {sum(v) / len(v):8.2f} "
                   f"{v[len(v) // 2]:8.2f} {100 * sum(v) / total:6.2f}")
    return "\n".join(out) + "\n"


def _counter(path: str, counter: str):
    """{dispatch id: (kernel name, grid size, value)} for one counter."""
    per = defaultdict(float)
    meta = {}
    for r in _rows(path):
        if r.get("counter_name", "").strip() != counter:
            continue
        d = int(r["dispatch_id"])
        per[d] += float(r["counter_value"])
        meta[d] = (r["kernel_name"], int(r.get("grid_size", 0) or 0))
    return {d: (meta[d][0], meta[d][1], v) for d, v in per.items()}


def traffic(fetch_csv: str, write_csv: str, kernel: str, copy_bytes: int):
    """Per-launch fetch and write bytes of `kernel` (short name; a '+' joins
    kernels launched together, whose sums are added), scaled by the copy."""
    res = {}
    for tag, path, cname in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        disp = _counter(path, cname)
        copies = [v for (n, g, v) in disp.values() if _COPY.search(n)]
        # the calibration copy is the largest copy dispatch of the run
        ref = max(copies) if copies else 0.0
        factor = copy_bytes / (ref * 1024.0) if ref > 0 else None
        total = 0.0
        for part in kernel.split("+"):
            vals = [v for (n, g, v) in disp.values() if short_name(n).split("<")[0] == part]
            if not vals:
                raise SystemExit(f"no dispatch of {part} in {path}")
            total += sum(vals) / len(vals)
        res[tag] = {"kib_per_launch": total, "copy_kib": ref, "factor": factor,
                    "bytes_per_launch": total * 1024.0 * factor if factor else None,
                    "dispatches": len([1 for (n, g, v) in disp.values()
                                       if short_name(n).split("<")[0] in kernel.split("+")])}
    return res


def _launch_key(r):
    wg = int(r.get("workgroup_size_x") or r.get("workgroup_size") or 1)
    g = int(r.get("grid_size_x") or r.get("grid_size") or 0) // max(wg, 1)
    return short_name(r["kernel_name"]).split("<")[0], g


def mfma_use(counter_csv: str, trace_csv: str, kernels) -> dict:
    """{(kernel, workgroups): {"util": %, "gflop": bf16 GFLOP, "us": avg
    duration}} from one ``--pmc MfmaUtil MfmaFlopsBF16`` run (per dispatch:
    the MFMA busy cycles over active cycles x SIMDs, in percent, and 512 x
    the bf16 MFMA op count) and the kernel trace of the same workload, whose
    average launch duration turns the FLOP into a rate."""
    per = defaultdict(lambda: defaultdict(list))
    meta = {}
    for r in _rows(counter_csv):
        key = _launch_key(r)
        if kernels and key[0] not in kernels:
            continue
        d = int(r["dispatch_id"])
        meta[d] = key
        per[d][r["counter_name"].strip()].append(float(r["counter_value"]))
    acc = defaultdict(lambda: defaultdict(list))
    for d, cs in per.items():
        if "MfmaUtil" in cs:   # a ratio: rows of one dispatch are averaged
            acc[meta[d]]["util"].append(sum(cs["MfmaUtil"]) / len(cs["MfmaUtil"]))
        if "MfmaFlopsBF16" in cs:
            acc[meta[d]]["gflop"].append(sum(cs["MfmaFlopsBF16"]) / 1e9)
    dur = defaultdict(list)
    for r in _rows(trace_csv):
        dur[_launch_key(r)].append((int(r["end_timestamp"]) - int(r["start_timestamp"])) / 1e3)
    out = {}
    for key, cs in acc.items():
        row = {k: sum(v) / len(v) for k, v in cs.items()}
        row["us"] = sum(dur[key]) / len(dur[key]) if dur.get(key) else float("nan")
        row["launches"] = max(len(v) for v in cs.values())
        out[key] = row
    return out


def mfma_summary(counter_csv: str, trace_csv: str, kernels, commands) -> str:
    res = mfma_use(counter_csv, trace_csv, kernels)
    out = ["# MFMA use per launch shape from rocprofv3 --pmc MfmaUtil MfmaFlopsBF16"]
    out += [f"command: {c}" for c in commands]
    out += ["MfmaUtil = MFMA busy cycles / (GPU active cycles x SIMDs), in percent;",
            "TFLOP/s = the launch's bf16 MFMA FLOP / its average duration in the kernel trace;",
            "of_peak against the dense bf16 MFMA peak, 2.5 PFLOP/s", "",
            f"{'kernel':16s} {'wgs':>6s} {'launches':>8s} {'MfmaUtil_%':>10s} {'GFLOP':>9s} "
            f"{'avg_us':>8s} {'TFLOP/s':>8s} {'of_peak':>8s}"]
    for (name, wg), r in sorted(res.items(), key=lambda kv: -kv[1].get("gflop", 0.0)):
        gf = r.get("gflop", float("nan"))
        tf = gf / r["us"] * 1e3 if r["us"] == r["us"] and r["us"] > 0 else float("nan")
        out.append(f"{name:16s} {wg:6d} {r['launches']:8d} {r.get('util', float('nan')):10.3f} "
                   f"{gf:9.4f} {r['us']:8.2f} {tf:8.2f} {tf / 2500.0:8.4f}")
    return "\n".join(out) + "\n"


def copy_overlap(trace_csv: str, copy_csv: str, kernels) -> dict:
    """{(kernel, workgroups): (mean us alone, launches, mean us with a copy in
    flight, launches)} from a run's kernel trace and memory-copy trace: a
    launch counts as "with a copy" when any copy's interval overlaps its own."""
    copies = sorted((int(r["start_timestamp"]), int(r["end_timestamp"])) for r in _rows(copy_csv))
    starts = [c[0] for c in copies]
    acc = defaultdict(lambda: ([], []))
    for r in _rows(trace_csv):
        key = _launch_key(r)
        if kernels and key[0] not in kernels:
            continue
        s0, s1 = int(r["start_timestamp"]), int(r["end_timestamp"])
        # copies starting before the launch ends; any of them ending after it starts overlaps
        k = bisect.bisect_left(starts, s1)
        hit = any(copies[j][1] > s0 for j in range(max(0, k - 64), k))
        acc[key][1 if hit else 0].append((s1 - s0) / 1e3)
    return {key: (sum(a) / len(a) if a else float("nan"), len(a),
                  sum(b) / len(b) if b else float("nan"), len(b))
            for key, (a, b) in acc.items()}


def overlap_summary(trace_csv: str, copy_csv: str, kernels, command: str) -> str:
    res = copy_overlap(trace_csv, copy_csv, kernels)
    n_copy = sum(1 for _ in _rows(copy_csv))
    out = ["# Kernel durations with and without a host-to-device copy in flight",
           f"command: {command}", f"memory copies in the trace: {n_copy}", "",
           f"{'kernel':16s} {'wgs':>6s} {'alone_us':>9s} {'n':>5s} {'with_copy_us':>12s} "
           f"{'n':>5s} {'delta_us':>8s}"]
    for (name, wg), (a, na, b, nb) in sorted(res.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        out.append(f"{name:16s} {wg:6d} {a:9.2f} {na:5d} {b:12.2f} {nb:5d} {b - a:8.2f}")
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--trace", help="the run's *_kernel_trace.csv: adds launches by grid")
    s.add_argument("--note", action="append", default=[])
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--kernel", action="append", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--json", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--command", action="append", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("counters")
    m.add_argument("trace")
    m.add_argument("--kernel", action="append", default=[])
    m.add_argument("--command", action="append", required=True)
    m.add_argument("--out", required=True)
    o = sub.add_parser("overlap")
    o.add_argument("trace")
    o.add_argument("copies")
    o.add_argument("--kernel", action="append", default=[])
    o.add_argument("--command", required=True)
    o.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "overlap":
        with open(a.out, "w") as f:
            f.write(overlap_summary(a.trace, a.copies, a.kernel, a.command))
        return
    if a.cmd == "mfma":
        with open(a.out, "w") as f:
            f.write(mfma_summary(a.counters, a.trace, a.kernel, a.command))
        return
    if a.cmd == "stats":
        with open(a.out, "w") as f:
            f.write(kernel_stats(a.csv, a.command))
            if a.trace:
                f.write("\nlaunches by kernel and grid (workgroups):\n")
                f.write(launches_by_grid(a.trace))
            for n in a.note:
                f.write(f"\n{n}\n")
        return
    try:
        with open(a.json) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    lines = ["# HBM traffic per launch from rocprofv3 --pmc (FETCH_SIZE, WRITE_SIZE)"]
    lines += [f"command: {c}" for c in a.command]
    lines.append(f"calibration: a device copy of {a.copy_bytes} bytes (reads and writes that many)")
    for k in a.kernel:
        r = traffic(a.fetch, a.write, k, a.copy_bytes)
        fb, wb = r["fetch"]["bytes_per_launch"], r["write"]["bytes_per_launch"]
        ent = {"bytes_per_launch": (fb + wb) if fb is not None and wb is not None else None,
               "fetch_bytes": fb, "write_bytes": wb,
               "fetch_factor": r["fetch"]["factor"], "write_factor": r["write"]["factor"],
               "source_hash": source_hash()}
        data.setdefault(a.workload, {})[k] = ent
        lines.append(f"{a.workload} {k}: fetch {r['fetch']['kib_per_launch']:.1f} KiB x "
                     f"{r['fetch']['factor']:.4f}, write {r['write']['kib_per_launch']:.1f} KiB x "
                     f"{r['write']['factor']:.4f} -> {ent['bytes_per_launch'] / 1e6:.3f} MB per launch "
                     f"({r['fetch']['dispatches']} dispatches; copy read {r['fetch']['copy_kib']:.0f} "
                     f"KiB, wrote {r['write']['copy_kib']:.0f} KiB)")
    with open(a.json, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
