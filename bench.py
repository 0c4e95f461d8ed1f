"""Benchmark of the multi-adapter LoRA delta on one MI355X.

A step is one pass of the whole delta over one heterogeneous batch: for the
full Mistral-7B-shaped stack (the default workload) that is 32 layers x 4
calls (qkv fused through y offsets, o, gate_up fused, down), i.e. all 224
(layer, projection) deltas y = base_out + s B (A x), with inputs already
resident in HBM.  The step is captured once in a HIP graph and replayed.

Prints one JSON line: tokens/s over the whole stack, achieved HBM GB/s of
the algorithmic bytes, the roofline of the dominant kernel (measured with
HIP events on the launch stream), and the CPU oracle's rate on the host.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0        # dense bf16 MFMA
METRIC = ("LoRA-delta tokens/s + achieved HBM GB/s (decode) / MFMA util (prefill), 1 GPU")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _core_elems(w):
    """float32 elements of one core: r_max^2 (full) or r_max (diag)."""
    return w.r_max * (w.r_max if w.sigma_kind == "full" else 1)


def _distinct_cores(w):
    tok = w.token_adapter()
    sig = np.full(w.num_tokens, -1)
    for s in range(w.num_segs):
        sig[w.seg_starts[s]:w.seg_starts[s + 1]] = w.seg_sigma[s]
    return len({int(j) for j, a in zip(sig, tok) if j >= 0 and a >= 0})


def algorithmic(w, layers=None):
    """Bytes and FLOPs the delta must move/do, each counted once: adapter
    bytes of the distinct (adapter, layer, projection) triples at true rank
    (for jointly compressed adapters: the shared bases plus the distinct
    cores, float32), each activation read once, y written once and its input
    (base_out or y) read once."""
    es = 2 if w.dtype == "bf16" else 4
    layers = range(w.num_layers) if layers is None else layers
    slots = w.token_slots()                          # [T][K]: a merge's K adapters a token
    touched = w.touched()
    act = int((slots >= 0).any(axis=1).sum())
    per_layer_adapter = sum(int(w.ranks[a]) * (p.h_in + p.h_out) for a in touched
                            for p in w.projs) * es
    if w.sigma_kind:
        per_layer_adapter += _distinct_cores(w) * len(w.projs) * _core_elems(w) * 4
    per_layer_x = sum(w.num_tokens * w.x_width(k) for k in w.x_keys()) * es
    per_layer_y = sum(w.num_tokens * p.h_out for p in w.projs) * es * 2
    flops = sum(2 * int(w.ranks[a]) * (p.h_in + p.h_out) for a in slots.ravel() if a >= 0
                for p in w.projs)
    n = len(list(layers))
    return {"adapter": per_layer_adapter * n, "x": per_layer_x * n, "y": per_layer_y * n,
            "bytes": (per_layer_adapter + per_layer_x + per_layer_y) * n, "flops": flops * n,
            "active_tokens": act}


def kernel_bytes(w, call, kind):
    """Algorithmic bytes of one shrink or expand launch for one call."""
    es = 2 if w.dtype == "bf16" else 4
    touched = w.touched()
    act = int((w.token_slots() >= 0).any(axis=1).sum())
    r_sum = sum(int(w.ranks[a]) for a in touched)
    # the float32 intermediate is not counted: it passes between the two
    # kernels as partial sums, which are not algorithmic bytes
    if kind == "shrink":
        h_in = w.projs[call[0]].h_in
        return r_sum * h_in * es * len(call) + act * h_in * es
    h_out = sum(w.projs[p].h_out for p in call)
    cores = _distinct_cores(w) * len(call) * _core_elems(w) * 4 if w.sigma_kind else 0
    return r_sum * h_out * es + 2 * w.num_tokens * h_out * es + cores


def traffic_from_profile(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    from heterogeneous_adapter_batching_amd.profiling import source_hash
    ent = data.get(workload, {}).get(kernel)
    if not ent or ent.get("source_hash") != source_hash():
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(w, blocks, layers, threads, min_seconds):
    """Time the oracle (as it is) on the host: whole passes over the sampled
    layers, repeated until at least `min_seconds` of oracle time."""
    import oracle
    inputs = []
    used = sorted({int(j) for j in w.seg_sigma if j >= 0}) if w.sigma_kind else []
    for l in layers:
        for p, pr in enumerate(w.projs):
            adapters = {a: (blocks[(a, l, p)][0], blocks[(a, l, p)][1], float(w.scales[a]))
                        for a in w.touched()}
            cores = None
            if w.sigma_kind:
                cores = np.zeros((w.n_cores,) + w.core(0, l, p).shape, np.float32)
                for j in used:
                    cores[j] = w.core(j, l, p)
            inputs.append((w.activation(l, pr.x_key), adapters,
                           w.base_out(l, p) if w.has_base else None, cores))
    t_total, passes = 0.0, 0
    while passes == 0 or t_total < min_seconds:
        for x, adapters, y_in, cores in inputs:
            t0 = time.perf_counter()
            if cores is not None:
                oracle.lora_delta_sigma(x, w.seg_starts, w.seg_adapter, w.seg_sigma, adapters,
                                        cores, w.sigma_kind, y_in, threads=threads)
            elif w.merge_ids is not None:
                oracle.lora_delta_merge(x, w.seg_starts, w.merge_ids, w.merge_w, adapters, y_in,
                                        threads=threads)
            else:
                oracle.lora_delta(x, w.seg_starts, w.seg_adapter, adapters, y_in,
                                  threads=threads)
            t_total += time.perf_counter() - t0
        passes += 1
    frac = len(layers) / w.num_layers
    # one thread, over the first layer's calls only (bounded)
    first = inputs[:len(w.projs)]
    t1 = 0.0
    for x, adapters, y_in, cores in first:
        t0 = time.perf_counter()
        if cores is not None:
            oracle.lora_delta_sigma(x, w.seg_starts, w.seg_adapter, w.seg_sigma, adapters,
                                    cores, w.sigma_kind, y_in, threads=1)
        elif w.merge_ids is not None:
            oracle.lora_delta_merge(x, w.seg_starts, w.merge_ids, w.merge_w, adapters, y_in,
                                    threads=1)
        else:
            oracle.lora_delta(x, w.seg_starts, w.seg_adapter, adapters, y_in, threads=1)
        t1 += time.perf_counter() - t0
    return {"value": passes * w.num_tokens * frac / t_total, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{passes} passes over {len(layers)} of {w.num_layers} layers x "
                      f"{len(w.projs)} projections, all {w.num_tokens} tokens, float32 oracle, "
                      f"{threads} OpenMP threads, {t_total:.2f} s",
            "single_thread": {"value": w.num_tokens / (t1 * w.num_layers), "unit": "tokens/s",
                              "sample": f"1 of {w.num_layers} layers, {t1:.2f} s"},
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _time_graph(fn, stream, warmup, steps):
    """ms per call of fn, captured in a HIP graph and replayed on stream."""
    import torch
    with torch.cuda.stream(stream):
        for _ in range(max(1, warmup)):
            fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        fn()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) / steps


def base_stack(w, stream, warmup, steps):
    """The base model's own projections on the same tokens: per layer and
    call, y = x W with W the call's (h_in, sum of h_out) bf16 weight, every
    layer with weights of its own (so nothing is served from cache across
    layers).  Returns (ms per pass, weight bytes)."""
    import torch
    gen = torch.Generator(device="cuda").manual_seed(w.seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    mats, xs, ys, nbytes = [], {}, [], 0
    for key in w.x_keys():
        xs[key] = torch.randn((w.num_tokens, w.x_width(key)), generator=gen, device="cuda",
                              dtype=torch.float32).to(dt)
    for _ in range(w.num_layers):
        for c in w.calls:
            h_in = w.projs[c[0]].h_in
            width = sum(w.projs[p].h_out for p in c)
            wt = torch.empty((h_in, width), device="cuda", dtype=dt).normal_(
                0.0, h_in ** -0.5, generator=gen)
            mats.append((w.projs[c[0]].x_key, wt))
            ys.append(torch.empty((w.num_tokens, width), device="cuda", dtype=dt))
            nbytes += wt.numel() * wt.element_size()

    def fn():
        for (key, wt), y in zip(mats, ys):
            torch.mm(xs[key], wt, out=y)

    ms = _time_graph(fn, stream, warmup, steps)
    del mats, xs, ys
    torch.cuda.empty_cache()
    return ms, nbytes


def sweep(args):
    """Delta time of the full stack against the number of distinct adapters
    in the batch and against the skew of a Zipf draw, beside the base model's
    own projection GEMMs on the same 128 decode tokens."""
    import torch
    import heterogeneous_adapter_batching_amd as hab
    from dataclasses import replace
    from synth import default_threads, sweep_assignments, sweep_stack
    from synth.device import DeviceWorkload

    hab.load()
    torch.cuda.set_device(0)
    w = sweep_stack(128)
    t0 = time.perf_counter()
    dw = DeviceWorkload(w, upload=np.arange(w.pool_size), threads=default_threads(),
                        plan_opts=plan_opts(args))
    torch.cuda.synchronize()
    log(f"[sweep] staged {w.name}: {time.perf_counter() - t0:.1f} s")
    stream = torch.cuda.Stream()
    base_ms, base_bytes = base_stack(w, stream, args.warmup, args.steps)
    log(f"[sweep] base projections: {base_ms:.4f} ms, {base_bytes / 1e9:.3f} GB of weights, "
        f"{base_bytes / (base_ms * 1e-3) / 1e9:.1f} GB/s")
    est_ms = base_bytes / (HBM_PEAK_GBS * 1e9) * 1e3
    points = []
    for label, params, ids in sweep_assignments(w.num_tokens, w.pool_size):
        wp = replace(w, seg_adapter=ids)
        dw.plan = hab.Plan(dw.pool, w.num_tokens, w.seg_starts, ids)
        dw.plan.upload(dw.max_proj)
        ms = _time_graph(dw.run_fused, stream, args.warmup, args.steps)
        alg = algorithmic(wp)
        st = dw.plan.stats()
        pt = {"label": label, **params, "distinct": int(len(wp.touched())),
              "active_tokens": alg["active_tokens"], "ms": round(ms, 5),
              "vs_base": round(ms / base_ms, 4), "vs_base_estimate": round(ms / est_ms, 4),
              "adapter_bytes": alg["adapter"], "bytes": alg["bytes"],
              "gbs": round(alg["bytes"] / (ms * 1e-3) / 1e9, 1),
              "groups": st["groups"], "max_block_tokens": st["max_block_tokens"]}
        points.append(pt)
        log(f"[sweep] {label:14s} distinct {pt['distinct']:4d}  {ms:.4f} ms  "
            f"x{pt['vs_base']:.3f} of base  adapter {alg['adapter'] / 1e9:.3f} GB  "
            f"{pt['gbs']:.0f} GB/s")
    out = {"metric": "LoRA-delta ms per step vs distinct adapters and Zipf skew, 1 GPU",
           "unit": "ms", "higher_is_better": False, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "dtype": w.dtype, "data": "synthetic",
           "config": {"workload": w.name, "description": w.description,
                      "tokens": w.num_tokens, "layers": w.num_layers, "mode": "graph"},
           "base": {"ms": round(base_ms, 5), "weight_bytes": base_bytes,
                    "estimate_ms_at_peak": round(est_ms, 5)},
           "points": points}
    if args.sweep_out:
        lines = ["# LoRA delta vs distinct adapters and Zipf skew (full stack, 128 decode tokens)",
                 f"command: python bench.py --sweep --steps {args.steps} --warmup {args.warmup} "
                 f"--sweep-out {args.sweep_out}",
                 f"base projections (torch.mm, bf16, graph): {base_ms:.4f} ms for "
                 f"{base_bytes / 1e9:.3f} GB of weights "
                 f"({base_bytes / (base_ms * 1e-3) / 1e9:.0f} GB/s); at 8 TB/s: {est_ms:.4f} ms",
                 "",
                 f"{'point':14s} {'distinct':>8s} {'groups':>6s} {'ms':>8s} {'x base':>7s} "
                 f"{'adapter GB':>10s} {'GB/s':>6s}"]
        for p in points:
            lines.append(f"{p['label']:14s} {p['distinct']:8d} {p['groups']:6d} {p['ms']:8.4f} "
                         f"{p['vs_base']:7.3f} {p['adapter_bytes'] / 1e9:10.3f} {p['gbs']:6.0f}")
        with open(args.sweep_out, "w") as f:
            f.write("\n".join(lines) + "\n")
    print(json.dumps(out), flush=True)


def exchange(args):
    """Adapter exchange on the full stack (rank-16 adapters, 32 layers x 7
    projections, about 84 MB packed each): the host-to-device rate of packed
    images from pinned memory, how much of that copy the delta hides, and a
    replay of a continuous decode batch whose requests come and go, served
    from a pool smaller than the adapters it sees."""
    import torch
    import heterogeneous_adapter_batching_amd as hab
    from synth import config, default_threads, zipf_probs
    from synth.device import host_weights, to_device
    from concurrent.futures import ThreadPoolExecutor

    hab.load()
    torch.cuda.set_device(0)
    w = config(4)
    h_in, h_out = [p.h_in for p in w.projs], [p.h_out for p in w.projs]
    desc = hab.api.make_desc(w.num_layers, h_in, h_out, w.r_max, w.dtype)
    ext = hab.extent_bytes(desc, 16)
    n_img = args.exchange_images

    def image(aid):
        A = [np.stack([host_weights(w.adapter_block(aid, l, p)[0], w.dtype)
                       for l in range(w.num_layers)]) for p in range(len(w.projs))]
        B = [np.stack([host_weights(w.adapter_block(aid, l, p)[1], w.dtype)
                       for l in range(w.num_layers)]) for p in range(len(w.projs))]
        img = torch.empty(ext, dtype=torch.uint8, pin_memory=True)
        hab.pack_adapter(desc, 16, A, B, out=img.numpy())
        return img

    t0 = time.perf_counter()
    with ThreadPoolExecutor(min(8, default_threads())) as ex:
        images = list(ex.map(image, range(n_img)))
    log(f"[exchange] {n_img} packed images of {ext / 1e6:.1f} MB in pinned memory: "
        f"{time.perf_counter() - t0:.1f} s")

    # activations and outputs of the stack
    calls = [tuple(c) for c in w.calls]
    y_offsets = []
    for c in calls:
        o, offs = 0, []
        for p in c:
            offs.append(o)
            o += w.projs[p].h_out
        y_offsets.append(offs)
    x = {(l, k): to_device(w.activation(l, k), w.dtype) for l in range(w.num_layers)
         for k in w.x_keys()}
    base = {(l, ci): to_device(np.concatenate([w.base_out(l, p) for p in c], axis=1), w.dtype)
            for l in range(w.num_layers) for ci, c in enumerate(calls)}
    y = {k: torch.empty_like(v) for k, v in base.items()}
    comp, copy = torch.cuda.Stream(), torch.cuda.Stream()

    def new_pool(slots):
        return hab.Pool(w.num_layers, h_in, h_out, w.r_max, w.dtype, slab_bytes=slots * ext,
                        max_slots=max(slots, 1))

    def launch(pool, plan):
        for l in range(w.num_layers):
            for ci, c in enumerate(calls):
                hab.sgmv_fused(pool, plan, l, c, y_offsets[ci], x[(l, w.projs[c[0]].x_key)],
                               y[(l, ci)], base[(l, ci)], stream=comp)

    def timed(fn, n):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t = time.perf_counter()
        e0.record(comp)
        fn(n)
        e1.record(comp)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, (time.perf_counter() - t) * 1e3 / n

    T = w.num_tokens
    starts = np.arange(T + 1, dtype=np.int32)
    out = {}

    # 1. copy rate: packed images into a pool on the copy stream, nothing else running
    pool = new_pool(n_img)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(copy)
    for i in range(n_img):
        pool.register_image(i, 16, 2.0, images[i], stream=copy)
    c1.record(copy)
    torch.cuda.synchronize()
    copy_ms = c0.elapsed_time(c1)
    h2d = n_img * ext / (copy_ms * 1e-3) / 1e9
    out["h2d_gbs"] = round(h2d, 2)
    out["copy_ms_per_adapter"] = round(copy_ms / n_img, 4)
    log(f"[exchange] host-to-device: {n_img} images in {copy_ms:.2f} ms = {h2d:.1f} GB/s")

    # 2. overlap: the step (a graph over 8 resident adapters) on the compute
    # stream while the copy stream uploads packed images into another pool;
    # both start from one event
    ids0 = (np.arange(T, dtype=np.int32) % 8)
    pool2 = new_pool(8)
    for i in range(8):
        pool2.register_image(i, 16, 2.0, images[i], stream=comp)
    plan2 = hab.Plan(pool2, T, starts, ids0)
    with torch.cuda.stream(comp):
        plan2.upload(3, stream=comp)
        launch(pool2, plan2)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=comp):
        launch(pool2, plan2)
    torch.cuda.synchronize()
    n_steps = args.exchange_steps
    step_ms = _time_graph(lambda: launch(pool2, plan2), comp, 3, n_steps)
    n_copy = max(1, int(round(n_steps * step_ms / (copy_ms / n_img))))
    sink = new_pool(4)
    live = []                  # ids in the sink pool; copies on one stream reuse extents in order

    def copies(n):
        for i in range(n):
            if len(live) == 4:
                sink.unregister(live.pop(0))
            live.append(1000 + i)
            sink.register_image(live[-1], 16, 2.0, images[i % n_img], stream=copy)

    def together(do_copy, do_comp):
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(comp)
        copy.wait_event(ev[0])
        if do_copy:
            copies(n_copy)
        ev[1].record(copy)
        with torch.cuda.stream(comp):
            if do_comp:
                for _ in range(n_steps):
                    graph.replay()
        ev[2].record(comp)
        torch.cuda.synchronize()
        while live:
            sink.unregister(live.pop(0))
        return max(ev[0].elapsed_time(ev[1]), ev[0].elapsed_time(ev[2]))

    t_c = together(False, True)
    t_x = together(True, False)
    t_o = together(True, True)
    eff = (t_c + t_x - t_o) / min(t_c, t_x)
    out["overlap"] = {"steps": n_steps, "copies": n_copy, "compute_ms": round(t_c, 3),
                      "copy_ms": round(t_x, 3), "both_ms": round(t_o, 3),
                      "efficiency": round(eff, 3),
                      "step_ms_alone": round(t_c / n_steps, 4),
                      "step_ms_with_copies": round(t_o / n_steps, 4)}
    log(f"[exchange] overlap: {n_steps} steps {t_c:.2f} ms alone, {n_copy} copies "
        f"{t_x:.2f} ms alone, {t_o:.2f} ms together (hidden {eff:.0%} of the shorter)")
    del graph, plan2, pool2, sink
    torch.cuda.synchronize()

    # 3. replay: 128 decode slots, `churn` requests replaced each step by
    # Zipf(1.1) draws over 1000 adapters (ids map onto the packed images)
    g = np.random.default_rng(11)
    p_zipf = zipf_probs(1000, 1.1)
    for churn in args.exchange_churn:
        seq, cur = [], g.choice(1000, T, p=p_zipf).astype(np.int32)
        for k in range(n_steps + 4):
            cur = cur.copy()
            cur[g.choice(T, churn, replace=False)] = g.choice(1000, churn, p=p_zipf)
            seq.append(cur)
        distinct = len({int(a) for s in seq for a in s})
        res = {}
        for mode, slots in (("resident", distinct), ("exchange", args.exchange_slots),
                            ("exchange_no_prefetch", args.exchange_slots)):
            pool3 = new_pool(slots)
            cache = hab.Cache(pool3, copy_stream=copy)
            for a in sorted({int(a) for s in seq for a in s}):
                cache.add(a, 16, 2.0, images[a % n_img])
            if mode == "resident":
                for k in range(len(seq)):
                    cache.prefetch(seq[k])
                torch.cuda.synchronize()

            # one plan re-planned in place for every batch, one workspace
            # sized for any batch of T tokens: nothing is allocated per step
            ws = torch.empty(pool3.workspace_bytes(T, T, 3), dtype=torch.uint8, device="cuda")
            plan_box = [None]

            def run(n, start, mode=mode, cache=cache, pool3=pool3, ws=ws, plan_box=plan_box):
                for k in range(start, start + n):
                    cache.acquire(seq[k], stream=comp)
                    # the next batch's adapters copy while this batch runs
                    # (this batch's are held, so they stay)
                    if mode == "exchange" and k + 1 < len(seq):
                        cache.prefetch(seq[k + 1])
                    # re-planning takes the pool as it is now, evictions
                    # included, so the rebuilt plan is current
                    pl = plan_box[0]
                    if pl is None:
                        pl = plan_box[0] = hab.Plan(pool3, T, starts, seq[k])
                    else:
                        pl.rebuild(T, starts, seq[k])
                    pl.upload(3, ws=ws, stream=comp)
                    launch(pool3, pl)
                    cache.release(stream=comp)

            run(4, 0)
            before = cache.stats()
            ms, wall = timed(lambda n: run(n, 4), n_steps)
            st = cache.stats()
            up = st["bytes_uploaded"] - before["bytes_uploaded"]
            acq = (st["hits"] - before["hits"]) + (st["misses"] - before["misses"])
            res[mode] = {"ms_per_step": round(ms, 4), "wall_ms_per_step": round(wall, 4),
                         "hit_rate": round((st["hits"] - before["hits"]) / max(acq, 1), 4),
                         "uploaded_mb_per_step": round(up / n_steps / 1e6, 2),
                         "evictions_per_step": round(
                             (st["evictions"] - before["evictions"]) / n_steps, 3),
                         "slots": slots}
            log(f"[exchange] churn {churn}, {mode:20s}: {ms:.3f} ms/step, "
                f"hit rate {res[mode]['hit_rate']:.3f}, "
                f"{res[mode]['uploaded_mb_per_step']:.0f} MB uploaded per step")
            del cache, pool3
            torch.cuda.synchronize()
        out[f"replay_churn_{churn}"] = {"distinct_adapters": distinct, **res}

    line = {"metric": "adapter exchange: H2D GB/s, overlap efficiency, replay step time, 1 GPU",
            "unit": "mixed", "n_gpus": 1, "steps": n_steps, "dtype": w.dtype,
            "data": "synthetic",
            "config": {"workload": "full_stack_bf16 exchange", "adapter_mb": round(ext / 1e6, 2),
                       "tokens": T, "layers": w.num_layers, "pool_slots": args.exchange_slots,
                       "mode": "eager"},
            **out}
    if args.sweep_out:
        with open(args.sweep_out, "w") as f:
            f.write(f"# Adapter exchange on the full stack (rank-16 adapters, {ext / 1e6:.1f} MB "
                    f"packed each; {T} decode tokens)\n")
            f.write(f"command: python bench.py --exchange --exchange-steps {n_steps} "
                    f"--sweep-out {args.sweep_out}\n\n")
            f.write(f"host-to-device, packed images from pinned memory: {out['h2d_gbs']} GB/s "
                    f"({out['copy_ms_per_adapter']} ms per adapter)\n")
            f.write("overlap (the step captured in a graph over 8 resident adapters, on the "
                    "compute stream; image copies on the copy stream; both start from one "
                    "event):\n")
            f.write(f"  {json.dumps(out['overlap'])}\n")
            f.write(f"replay ({T} decode slots, `churn` requests replaced per step by Zipf(1.1) "
                    f"draws over 1000 adapters; eager launches; one plan rebuilt in place per "
                    f"batch into one workspace; pool of {args.exchange_slots} adapters):\n")
            for churn in args.exchange_churn:
                r = out[f"replay_churn_{churn}"]
                f.write(f"  replay_churn_{churn}: distinct adapters {r['distinct_adapters']}\n")
                for mode in ("resident", "exchange", "exchange_no_prefetch"):
                    f.write(f"    {mode:22s} {json.dumps(r[mode])}\n")
    print(json.dumps(line), flush=True)


def step_metrics(w, ms):
    """tokens/s, GB/s and TFLOP/s of one step of `ms` milliseconds, each with
    its roofline fraction (HBM for bytes; for FLOPs both the MFMA peak and the
    attainable roof min(MFMA peak, intensity x HBM peak))."""
    alg = algorithmic(w)
    tflops = alg["flops"] / (ms * 1e-3) / 1e12
    gbs = alg["bytes"] / (ms * 1e-3) / 1e9
    attain = min(BF16_PEAK_TFLOPS, alg["flops"] / alg["bytes"] * HBM_PEAK_GBS / 1e3)
    return {"ms_per_step": round(ms, 5), "tokens_per_s": round(w.num_tokens / (ms * 1e-3), 1),
            "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "tflops": round(tflops, 3), "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 5),
            "attainable_tflops": round(attain, 2), "attainable_frac": round(tflops / attain, 4),
            "algorithmic_bytes_per_step": alg["bytes"], "flops_per_step": alg["flops"]}


def make_flush(mib):
    """A buffer that evicts the caches when read: written once here, so that
    reading it before a step leaves the 256 MB memory-side cache and the L2s
    holding its clean lines and none of the step's data.  (Writing it before
    each step instead would leave them full of dirty lines, whose write-back
    the step would pay: a cold 32 MB read runs at 2.2 TB/s after a 1 GiB
    write and at 3.8 TB/s after a 1 GiB read.)"""
    import torch
    if mib <= 0:
        return None
    buf = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    torch.cuda.synchronize()
    return buf


def clear_caches(flush):
    """Read the whole flush buffer (a reduction to one value)."""
    flush.view(torch_int32()).max()


def torch_int32():
    import torch
    return torch.int32


def timed_steps(step, stream, steps, flush):
    """Mean ms per step and the sorted single-step times.  Without a flush
    buffer the steps run back to back between two events (and again, each
    between its own events, for the spread); with one, each step runs alone
    between its own events after a read of the whole flush buffer."""
    import torch
    if flush is None:
        with torch.cuda.stream(stream):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                step()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
            evs[0].record(stream)
            for i in range(steps):
                step()
                evs[i + 1].record(stream)
            torch.cuda.synchronize()
        return ms, np.sort([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)])
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(steps)]
        for ea, eb in pairs:
            clear_caches(flush)
            ea.record(stream)
            step()
            eb.record(stream)
        torch.cuda.synchronize()
    per_step = np.sort([ea.elapsed_time(eb) for ea, eb in pairs])
    return float(per_step.mean()), per_step


def capture(fn, stream, warmup):
    """fn captured in a HIP graph after warm-up runs; returns the graph."""
    import torch
    with torch.cuda.stream(stream):
        for _ in range(max(1, warmup)):
            fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        fn()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            graph.replay()
    torch.cuda.synchronize()
    return graph


def plan_opts(args):
    """The plan options given on the command line (the library's defaults
    for the others)."""
    return {k: v for k, v in (("long_group", args.long_group), ("long_batch", args.long_batch),
                              ("shrink_groups", args.shrink_groups),
                              ("prefill_groups", args.prefill_groups)) if v is not None}


def other_config(ci, args, stream, flush):
    """The step of a smaller workload (a parity configuration), timed in a
    graph, each step after a cache flush (its data would otherwise sit in
    the 256 MB cache from the step before)."""
    import torch
    from synth import config, default_threads
    from synth.device import DeviceWorkload
    w = config(ci)
    t0 = time.perf_counter()
    dw = DeviceWorkload(w, threads=default_threads(), plan_opts=plan_opts(args))
    graph = capture(dw.run_fused, stream, args.warmup)
    ms, per_step = timed_steps(graph.replay, stream, args.steps, flush)
    out = {"workload": w.name, "description": w.description, "tokens": w.num_tokens,
           "distinct_adapters": int(len(w.touched())), "plan": dw.plan.stats(),
           "flush_mib_between_steps": (flush.numel() >> 20) if flush is not None else 0,
           "flush": "read",
           "step_ms_p10_p50_p90": [round(float(np.quantile(per_step, q)), 5)
                                   for q in (0.1, 0.5, 0.9)], **step_metrics(w, ms)}
    log(f"[bench] {w.name}: {ms:.4f} ms/step ({time.perf_counter() - t0:.1f} s with staging), "
        f"{out['hbm_frac']:.3f} of HBM peak, {out['attainable_frac']:.3f} of the attainable roof")
    del graph, dw
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def cost_floor(args, stream):
    """The flat part of the cost sweep: the full stack's 128 decode tokens
    served from 1 and from 16 distinct rank-16 adapters (token t takes t mod
    d), graph-timed back to back, beside no adapter at all (the launches and
    the copy of base_out into y)."""
    import torch
    import heterogeneous_adapter_batching_amd as hab
    from synth import default_threads, sweep_stack
    from synth.device import DeviceWorkload
    w = sweep_stack(16)
    t0 = time.perf_counter()
    dw = DeviceWorkload(w, upload=np.arange(w.pool_size), threads=default_threads(),
                        plan_opts=plan_opts(args))
    out = {"workload": w.name, "steps": args.steps}
    for d in (0, 1, 16):
        ids = np.full(w.num_tokens, -1, np.int32) if d == 0 else \
            (np.arange(w.num_tokens) % d).astype(np.int32)
        dw.plan = hab.Plan(dw.pool, w.num_tokens, w.seg_starts, ids)
        dw.plan.upload(dw.max_proj)
        out[f"distinct_{d}_ms"] = round(_time_graph(dw.run_fused, stream, args.warmup,
                                                     args.steps), 5)
    log(f"[bench] cost floor (0, 1, 16 distinct adapters): {out['distinct_0_ms']:.4f}, "
        f"{out['distinct_1_ms']:.4f}, {out['distinct_16_ms']:.4f} ms per step "
        f"({time.perf_counter() - t0:.1f} s with staging)")
    del dw
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def copy_ceiling(nbytes, launches, stream):
    """GB/s of a plain device copy moving `nbytes` per launch (half read,
    half written), `launches` copies back to back in a graph: the ceiling
    of a kernel of that size in the step's launch pattern."""
    import torch
    n = max(1, int(nbytes) // 4)                 # bf16 elements read per copy
    src = torch.ones(n * launches, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)

    def fn():
        for i in range(launches):
            dst[i * n:(i + 1) * n].copy_(src[i * n:(i + 1) * n])
    ms = _time_graph(fn, stream, 3, 10)
    del src, dst
    return 4 * n / (ms * 1e-3 / launches) / 1e9, ms * 1e3 / launches


def copy_step(sizes, stream):
    """ms of a graph of plain device copies, one per kernel launch of the
    step, each moving that launch's algorithmic bytes (half read, half
    written), in the step's order: the step's ceiling if every kernel ran
    at the speed of a copy of its size in this launch pattern."""
    import torch
    halves = [max(1, int(b) // 4) for b in sizes]     # bf16 elements read per copy
    total = sum(halves)
    src = torch.ones(total, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    offs = np.concatenate([[0], np.cumsum(halves)])

    def fn():
        for i in range(len(halves)):
            dst[offs[i]:offs[i + 1]].copy_(src[offs[i]:offs[i + 1]])
    ms = _time_graph(fn, stream, 3, 10)
    del src, dst
    return ms


def plan_cost(dw, stream, reps=200):
    """Host cost of planning a new batch: lora_plan_rebuild then
    lora_plan_upload into one workspace sized for any batch of the step's
    size, alternating two batches over the same adapters.  Returns the plan
    (uploaded), its workspace and microseconds per rebuild + upload."""
    import torch
    w = dw.w
    mp = dw.max_proj
    ws = torch.empty(dw.pool.workspace_bytes(w.num_tokens, w.num_segs, mp), dtype=torch.uint8,
                     device="cuda")
    ids = [np.asarray(w.seg_adapter, np.int32),
           np.random.default_rng(7).permutation(np.asarray(w.seg_adapter, np.int32))]
    plan = dw.plan
    for _ in range(5):
        plan.rebuild(w.num_tokens, w.seg_starts, ids[0]).upload(mp, ws=ws, stream=stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(reps):
        plan.rebuild(w.num_tokens, w.seg_starts, ids[i % 2]).upload(mp, ws=ws, stream=stream)
    us = (time.perf_counter() - t0) * 1e6 / reps
    torch.cuda.synchronize()
    return plan, ws, ids, us


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=4,
                    help="0..4 (default 4: the full stack); 5, 6: the full stack served from "
                         "jointly compressed adapters with full / diagonal cores; 7: the full "
                         "stack with each request merging 2 adapters")
    ap.add_argument("--mode", choices=("graph", "eager"), default="graph")
    ap.add_argument("--cpu-layers", type=int, default=-1,
                    help="layers of the CPU-oracle sample (-1: all, 0: skip)")
    ap.add_argument("--flush-mib", type=int, default=-1,
                    help="MiB written between timed steps, outside the timed events, so that "
                         "a step does not find the last step's data in the 256 MB Infinity "
                         "Cache or the L2s; -1: 1024 when a step moves under 1 GiB, else 0")
    ap.add_argument("--kernel-reps", type=int, default=5,
                    help="event-timed passes for the per-kernel roofline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum oracle time of the CPU baseline")
    ap.add_argument("--copy-mib", type=int, default=2048,
                    help="size of the device-copy bandwidth reference (0: skip)")
    ap.add_argument("--configs", type=int, nargs="*", default=[1, 2, 3],
                    help="smaller workloads also timed (flushed) and reported under 'configs'")
    ap.add_argument("--cost-floor", type=int, default=1,
                    help="with the full stack, also time it from 0, 1 and 16 distinct adapters "
                         "(the flat part of the cost sweep) under 'cost_floor' (0: skip)")
    for opt, what in (("long-group", "tokens that make a group long (the prompt kernel)"),
                      ("long-batch", "long groups' tokens a batch needs to use the prompt kernel"),
                      ("shrink-groups", "workgroups a decode shrink launch aims for"),
                      ("prefill-groups", "workgroups a prompt launch aims for")):
        ap.add_argument(f"--{opt}", type=int, default=None,
                        help=f"plan option: {what} (default: the library's)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the step: delta time vs distinct adapters and Zipf skew")
    ap.add_argument("--sweep-out", default=None, help="text summary of the sweep")
    ap.add_argument("--exchange", action="store_true",
                    help="instead of the step: adapter exchange rates and a replay")
    ap.add_argument("--exchange-images", type=int, default=24,
                    help="distinct packed adapters in pinned host memory")
    ap.add_argument("--exchange-steps", type=int, default=30)
    ap.add_argument("--exchange-slots", type=int, default=96,
                    help="pool capacity (adapters) of the replay")
    ap.add_argument("--exchange-churn", type=int, nargs="+", default=[1, 4],
                    help="requests replaced per step in the replay")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the delta "
              "shards over GPUs by request with no exchange between them, so one GPU's "
              "throughput is the figure)", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        return sweep(args)
    if args.exchange:
        return exchange(args)

    import torch
    import heterogeneous_adapter_batching_amd as hab
    from synth import config, default_threads
    from synth.device import DeviceWorkload

    hab.load()
    torch.cuda.set_device(0)
    if args.workload in (5, 6):
        from synth import jd_full_stack
        w = jd_full_stack("full" if args.workload == 5 else "diag")
    elif args.workload == 7:
        from synth import merge_full_stack
        w = merge_full_stack(2)
    else:
        w = config(args.workload)
    threads = min(16, os.cpu_count() or 1)
    cpu_layers = list(range(w.num_layers)) if args.cpu_layers < 0 else list(
        range(min(args.cpu_layers, w.num_layers)))
    keep = {}

    def on_block(aid, l, p, a, b):
        if l in cpu_layers:
            keep[(aid, l, p)] = (a, b)

    t0 = time.perf_counter()
    dw = DeviceWorkload(w, on_block=on_block, threads=default_threads(),
                        plan_opts=plan_opts(args))
    torch.cuda.synchronize()
    log(f"[bench] staged {w.name}: {time.perf_counter() - t0:.1f} s, "
        f"plan {dw.plan.stats()}")
    alg = algorithmic(w)
    # a call is one prefill launch for a batch of long groups only, else a
    # shrink and an expand launch
    launches = (1 if dw.plan.stats()["max_block_tokens"] > 16 else 2) * len(dw.layers) * \
        len(dw.calls)

    stream = torch.cuda.Stream()
    graph = capture(dw.run_fused, stream, args.warmup) if args.mode == "graph" else None
    step = graph.replay if graph is not None else dw.run_fused

    # A step that moves less than the caches hold would find the last step's
    # data there: such steps are timed one by one, each after a flush write.
    flush_mib = args.flush_mib if args.flush_mib >= 0 else (
        1024 if alg["bytes"] < (1 << 30) else 0)
    flush = make_flush(flush_mib)
    ms, per_step = timed_steps(step, stream, args.steps, flush)
    log(f"[bench] {args.mode}: {ms:.4f} ms/step" +
        (f", each step after a {flush_mib} MiB flush" if flush is not None else ""))
    quant = {q: round(float(np.quantile(per_step, v)), 5)
             for q, v in (("p10", 0.1), ("p50", 0.5), ("p90", 0.9))}

    # eager step time for reference (Python + C launch path, no graph)
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e2.record(stream)
        for _ in range(max(3, args.steps // 5)):
            dw.run_fused(stream=stream)
        e3.record(stream)
        torch.cuda.synchronize()
    eager_ms = e2.elapsed_time(e3) / max(3, args.steps // 5)

    # Per-batch planning on the measured path: a serving loop plans every
    # step (the batch changes).  The host cost of rebuild + upload, and an
    # eager step that plans its batch first, alternating two batches.
    plan_us = rebuild_ms = None
    if w.merge_ids is None:             # a merge plan is built, not rebuilt in place
        graph_plan = dw.plan
        plan, plan_ws, plan_ids, plan_us = plan_cost(dw, stream)
        log(f"[bench] plan rebuild + upload: {plan_us:.1f} us on the host")
        # three timed runs of n_rb re-planned steps, the median reported; the
        # garbage collector is held off meanwhile, as the host enqueues the
        # step's launches from Python
        n_rb = max(10, args.steps // 2)
        runs = []
        with torch.cuda.stream(stream):
            for i in range(3):   # untimed: the first re-planned steps of the process
                plan.rebuild(w.num_tokens, w.seg_starts, plan_ids[i % 2]).upload(
                    dw.max_proj, ws=plan_ws, stream=stream)
                dw.run_fused(stream=stream)
            torch.cuda.synchronize()
            gc_was = gc.isenabled()
            gc.disable()
            try:
                for _ in range(3):
                    e4, e5 = (torch.cuda.Event(enable_timing=True),
                              torch.cuda.Event(enable_timing=True))
                    t_rb = time.perf_counter()
                    e4.record(stream)
                    for i in range(n_rb):
                        plan.rebuild(w.num_tokens, w.seg_starts, plan_ids[i % 2]).upload(
                            dw.max_proj, ws=plan_ws, stream=stream)
                        dw.run_fused(stream=stream)
                    e5.record(stream)
                    torch.cuda.synchronize()
                    runs.append((e4.elapsed_time(e5) / n_rb,
                                 (time.perf_counter() - t_rb) * 1e3 / n_rb))
            finally:
                if gc_was:
                    gc.enable()
        rebuild_ms, t_rb = sorted(runs)[1]
        log(f"[bench] eager step planning its batch first: {rebuild_ms:.4f} ms "
            f"(host {t_rb:.4f} ms per step)")
        plan.rebuild(w.num_tokens, w.seg_starts, w.seg_adapter).upload(dw.max_proj, ws=plan_ws,
                                                                       stream=stream)
        torch.cuda.synchronize()

    # Per-kernel durations, launched back to back (a full queue, as in the
    # step), between two events on the launch stream.  Decode: the step's
    # two kernels, as passes over every (layer, call) of the shrink alone
    # and of the shrink then the expand (sgmv_fused's two kernels as separate
    # calls, in the step's order); the expand's duration is the pair's less
    # the shrink's.  A batch of long groups only: each call is one launch of
    # the prefill kernel, timed as passes of sgmv_fused.
    n_launch = len(dw.layers) * len(dw.calls)
    prefill = dw.plan.stats()["max_block_tokens"] > 16

    def one_pass(kind):
        for l in dw.layers:
            for ci, c in enumerate(dw.calls):
                x = dw.x[(l, w.projs[c[0]].x_key)]
                if kind == "prefill":
                    if dw.sigma is not None:
                        hab.sgmv_fused_sigma(dw.pool, dw.plan, l, c, dw.y_offsets[ci], x,
                                             dw.sigma, w.sigma_kind, dw.y[(l, ci)],
                                             dw.base.get((l, ci)), stream=stream)
                    else:
                        hab.sgmv_fused(dw.pool, dw.plan, l, c, dw.y_offsets[ci], x,
                                       dw.y[(l, ci)], dw.base.get((l, ci)), stream=stream)
                    continue
                hab.sgmv_shrink_partials(dw.pool, dw.plan, l, c, x, stream=stream)
                if kind == "shrink":
                    continue
                if dw.sigma is not None:
                    hab.sgmv_expand_partials_sigma(dw.pool, dw.plan, l, c, dw.y_offsets[ci],
                                                   dw.sigma, w.sigma_kind, dw.y[(l, ci)],
                                                   dw.base.get((l, ci)), stream=stream)
                else:
                    hab.sgmv_expand_partials(dw.pool, dw.plan, l, c, dw.y_offsets[ci],
                                             dw.y[(l, ci)], dw.base.get((l, ci)), stream=stream)

    tot = {}
    with torch.cuda.stream(stream):
        for kind in (("prefill",) if prefill else ("shrink", "pair")):
            one_pass(kind)                                   # warm
            torch.cuda.synchronize()
            if flush is None:
                ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                ea.record(stream)
                for _ in range(args.kernel_reps):
                    one_pass(kind)
                eb.record(stream)
                torch.cuda.synchronize()
                tot[kind] = ea.elapsed_time(eb)
            else:                                            # each pass after a flush
                pairs = [(torch.cuda.Event(enable_timing=True),
                          torch.cuda.Event(enable_timing=True)) for _ in range(args.kernel_reps)]
                for ea, eb in pairs:
                    clear_caches(flush)
                    ea.record(stream)
                    one_pass(kind)
                    eb.record(stream)
                torch.cuda.synchronize()
                tot[kind] = sum(ea.elapsed_time(eb) for ea, eb in pairs)
    if not prefill:
        tot["expand"] = tot["pair"] - tot["shrink"]
        tot.pop("pair")
    us = {kind: t * 1e3 / (args.kernel_reps * n_launch) for kind, t in tot.items()}
    kern = {}
    kinds = ("prefill",) if prefill else ("shrink", "expand", "fused")
    if not prefill:
        us["fused"] = us["shrink"] + us["expand"]
    for kind in kinds:
        parts = ("shrink", "expand") if kind in ("fused", "prefill") else (kind,)
        bpl = sum(kernel_bytes(w, c, k) for c in dw.calls for k in parts) / len(dw.calls)
        kern[kind] = {"avg_us": us[kind], "gbs": bpl / (us[kind] * 1e-6) / 1e9,
                      "alg_bytes_per_launch": bpl}
    if prefill:
        dom, kname = "prefill", "k_prefill"
    else:
        dom = "expand" if kern["expand"]["avg_us"] >= kern["shrink"]["avg_us"] else "shrink"
        kname = {"shrink": "k_shrink",
                 "expand": "k_expand_merge" if w.merge_ids is not None else "k_expand_decode"}[dom]
    traffic = traffic_from_profile(kname, w.name)
    roof = {"bound": "hbm", "achieved": round(kern[dom]["gbs"], 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(kern[dom]["gbs"] / HBM_PEAK_GBS, 4),
            "traffic": traffic, "kernel": kname,
            "avg_launch_us": round(kern[dom]["avg_us"], 3),
            "alg_bytes_per_launch": int(kern[dom]["alg_bytes_per_launch"])}
    log(f"[bench] kernels: {json.dumps(kern)}")

    # the ceiling of a kernel of this size in this launch pattern: a plain
    # copy moving the same bytes per launch, as many launches back to back
    if flush is None and args.copy_mib > 0:
        cgbs, cus = copy_ceiling(kern[dom]["alg_bytes_per_launch"], n_launch, stream)
        roof["copy_same_bytes_gbs"] = round(cgbs, 1)
        roof["copy_same_bytes_us"] = round(cus, 3)
        roof["frac_of_copy_same_bytes"] = round(kern[dom]["gbs"] / cgbs, 4)
        log(f"[bench] copy of {kern[dom]['alg_bytes_per_launch'] / 1e6:.1f} MB per launch, "
            f"{n_launch} back to back: {cus:.2f} us, {cgbs:.0f} GB/s")

    # the step as copies: every launch of the step replaced by a copy of its
    # algorithmic bytes, in the same order, in a graph
    copy_step_ms = None
    if flush is None and args.copy_mib > 0:
        sizes = [kernel_bytes(w, c, k) for _ in dw.layers for c in dw.calls
                 for k in ("shrink", "expand")]
        copy_step_ms = copy_step(sizes, stream)
        log(f"[bench] the step as {len(sizes)} copies of its launches' bytes: "
            f"{copy_step_ms:.4f} ms ({alg['bytes'] / (copy_step_ms * 1e-3) / 1e9:.0f} GB/s)")

    # device copy bandwidth: a second, measured denominator
    copy_gbs = None
    if args.copy_mib > 0:
        nel = args.copy_mib * (1 << 20) // 2
        src = torch.empty(nel, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            dst.copy_(src)
            torch.cuda.synchronize()
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            for _ in range(5):
                dst.copy_(src)
            c1.record(stream)
            torch.cuda.synchronize()
        copy_gbs = 2 * nel * 2 * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
        del src, dst
        log(f"[bench] device copy of {args.copy_mib} MiB: {copy_gbs:.1f} GB/s (read + write)")

    cpu = None
    if args.cpu_layers != 0 and keep:
        cpu = cpu_baseline(w, keep, cpu_layers, threads, args.cpu_seconds)
        log(f"[bench] cpu baseline: {cpu}")
    keep.clear()

    # the smaller workloads, each step after a 1 GiB flush
    del graph
    step_opts = dw.plan.opts()
    configs = {}
    if args.workload == 4 and args.configs:
        del dw, plan, plan_ws, graph_plan
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        cflush = make_flush(1024)
        for ci in args.configs:
            configs[f"config{ci}"] = other_config(ci, args, stream, cflush)
        del cflush
    floor = cost_floor(args, stream) if args.workload == 4 and args.cost_floor else None

    m = step_metrics(w, ms)
    out = {
        "metric": METRIC, "value": m["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": m["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16"
        if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "description": w.description,
                   "tokens": w.num_tokens, "layers": w.num_layers,
                   "projections": [p.name for p in w.projs],
                   "calls_per_layer": len(w.calls), "kernel_launches_per_step": launches,
                   "distinct_adapters": int(len(w.touched())), "mode": args.mode,
                   "flush_mib_between_steps": flush_mib, "flush": "read",
                   "plan_opts": step_opts},
        **{k: v for k, v in m.items() if k not in ("ms_per_step", "tokens_per_s")},
        "step_ms_quantiles": quant,
        "eager_ms_per_step": round(eager_ms, 5),
        # a serving loop plans each batch: host microseconds of rebuild +
        # upload, and the eager step that does so first
        "plan_us": None if plan_us is None else round(plan_us, 2),
        "eager_replan_ms_per_step": None if rebuild_ms is None else round(rebuild_ms, 5),
        "kernels": {k: {kk: round(vv, 3) for kk, vv in d.items()} for k, d in kern.items()},
        "copy_gbs": round(copy_gbs, 1) if copy_gbs else None,
        # the same bytes per launch moved by plain copies in the same order
        "copy_step_ms": round(copy_step_ms, 5) if copy_step_ms else None,
        "frac_of_copy_step": round(copy_step_ms / ms, 4) if copy_step_ms else None,
        "roofline": roof, "cpu_baseline": cpu, "configs": configs, "cost_floor": floor,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
