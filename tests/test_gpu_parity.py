"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

The contract tolerance is max|y_gpu - y_ref| <= 1e-2 * max|y_ref| + 1e-3 per
output tensor, for bf16 inputs with float32 accumulation.  On small cases a
much tighter bound is also enforced: the GPU must be as accurate as float32
arithmetic itself (a rounding-error bound for the two sums, the scale and the
add, plus the single rounding of y to bf16), measured against the float64
oracle.  Gather, segment indexing, padding, permutation and determinism are
checked bit for bit.
"""
import dataclasses
import os
import sys

import numpy as np
import pytest

import oracle
from synth import config, mixed_case, random_case, Proj
from synth.device import DeviceWorkload, from_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import heterogeneous_adapter_batching_amd as hab
    hab.load()


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def contract_check(y_gpu, y_ref, what):
    assert y_gpu.shape == y_ref.shape, what
    if y_ref.size == 0:
        return 0.0, 1e-3
    tol = 1e-2 * float(np.abs(y_ref).max()) + 1e-3
    err = float(np.abs(y_gpu.astype(np.float64) - y_ref).max())
    assert err <= tol, f"{what}: max|diff| {err:.3e} > tol {tol:.3e}"
    return err, tol


def oracle_ref(w, layer, p, acc="f32", threads=8):
    return oracle.workload_call(w, layer, p, acc=acc, threads=threads)


def tight_bound(w, layer, p, out_bf16):
    """Per-element bound for a float32 evaluation of y_in + s B (A x) in any
    summation order (|error| <= gamma_n * sum|terms| per sum, with 2u per
    operation to allow a non-nearest internal rounding), plus the final
    rounding of y to the output type."""
    u = 2.0 ** -23
    pr = w.projs[p]
    x = w.activation(layer, pr.x_key).astype(np.float64)
    tok = w.token_adapter()
    y_in = w.base_out(layer, p).astype(np.float64) if w.has_base else np.zeros(
        (w.num_tokens, pr.h_out))
    bound = np.zeros((w.num_tokens, pr.h_out))
    for t in range(w.num_tokens):
        i = int(tok[t])
        if i < 0:
            continue
        a, b = (m.astype(np.float64) for m in w.adapter_block(i, layer, p))
        s = abs(float(w.scales[i]))
        r = a.shape[0]
        absv = np.abs(a) @ np.abs(x[t])
        ga = (pr.h_in + 64) * u
        gb = (3 * r + 4) * u
        e = s * (ga * (np.abs(b) @ absv) + gb * (np.abs(b) @ absv)) + u * (
            np.abs(y_in[t]) + s * (np.abs(b) @ absv))
        bound[t] = e
    y64 = oracle_ref(w, layer, p, acc="f64")
    out_r = (2.0 ** -8 if out_bf16 else 2.0 ** -24) * (np.abs(y64) + bound)
    return y64, 1.01 * (bound + out_r) + 1e-30


def check_workload(dw, tight=False, threads=8):
    w = dw.w
    for l in dw.layers:
        for p in range(len(w.projs)):
            got = dw.output(l, p)
            ref = oracle_ref(w, l, p, threads=threads)
            contract_check(got, ref, f"{w.name} layer {l} proj {w.projs[p].name}")
            if tight:
                y64, bnd = tight_bound(w, l, p, w.dtype == "bf16")
                viol = np.abs(got.astype(np.float64) - y64) > bnd
                assert not viol.any(), (
                    f"{w.name} {w.projs[p].name}: {int(viol.sum())} elements outside the "
                    f"float32 bound, worst {np.max(np.abs(got - y64) - bnd):.3e}")


# ------------------------------------------------------------- workloads ----
@pytest.mark.parametrize("ci", [0, 1, 2, 3])
def test_workload_parity(ci):
    w = config(ci)
    log(f"[parity] workload {ci} {w.name}")
    dw = DeviceWorkload(w, slab_fill=0xFF if ci == 3 else None)   # NaN over untouched extents
    dw.zero_outputs()
    dw.run_fused()
    torch.cuda.synchronize()
    check_workload(dw, tight=ci in (0, 1))


def test_full_stack_parity():
    """The 32-layer x 7-projection stack, in the launch pattern the benchmark
    times (4 calls per layer: qkv, o, gate_up, down), every output checked."""
    w = config(4)
    log("[parity] full stack (workload 4)")
    refs = {}
    pending = {}
    touched = w.touched()

    def on_block(aid, l, p, a, b):
        pending.setdefault((l, p), {})[aid] = (a, b, float(w.scales[aid]))
        if len(pending[(l, p)]) == len(touched):
            pr = w.projs[p]
            refs[(l, p)] = oracle.lora_delta(w.activation(l, pr.x_key), w.seg_starts,
                                             w.seg_adapter, pending.pop((l, p)),
                                             w.base_out(l, p), threads=16)
            if p == len(w.projs) - 1:
                log(f"[parity] full stack: layer {l} staged and oracle done")

    dw = DeviceWorkload(w, on_block=on_block)
    dw.run_fused()
    torch.cuda.synchronize()
    worst = 0.0
    for (l, p), ref in refs.items():
        got = dw.output(l, p)
        err, tol = contract_check(got, ref, f"layer {l} proj {w.projs[p].name}")
        # the delta alone, to a tolerance scaled by the delta (plus bf16 rounding of y)
        d_ref = ref - w.base_out(l, p)
        lim = 1e-2 * np.abs(d_ref).max() + 1e-3 + 2.0 ** -8 * np.abs(ref)
        assert np.all(np.abs(got - ref) <= lim), f"delta check layer {l} proj {p}"
        worst = max(worst, err / tol)
    assert len(refs) == 32 * 7
    log(f"[parity] full stack worst err/tol {worst:.3f}")


def test_merge_full_stack_parity():
    """The full stack with every request merging 2 adapters (the merged
    workload the benchmark times: one shrink over every (token, slot) row and
    one merge expand per call), every output of the 32 layers x 7
    projections against the oracle's merge."""
    from synth import merge_full_stack
    w = merge_full_stack(2)
    log("[parity] merged full stack (2 adapters a request)")
    refs, pending = {}, {}
    touched = w.touched()

    def on_block(aid, l, p, a, b):
        pending.setdefault((l, p), {})[aid] = (a, b, float(w.scales[aid]))
        if len(pending[(l, p)]) == len(touched):
            pr = w.projs[p]
            refs[(l, p)] = oracle.lora_delta_merge(w.activation(l, pr.x_key), w.seg_starts,
                                                   w.merge_ids, w.merge_w, pending.pop((l, p)),
                                                   w.base_out(l, p), threads=16)

    dw = DeviceWorkload(w, on_block=on_block)
    assert dw.plan.stats()["max_block_tokens"] <= 4
    dw.run_fused()
    torch.cuda.synchronize()
    worst = 0.0
    for (l, p), ref in refs.items():
        got = dw.output(l, p)
        err, tol = contract_check(got, ref, f"merged layer {l} proj {w.projs[p].name}")
        d_ref = ref - w.base_out(l, p)
        lim = 1e-2 * np.abs(d_ref).max() + 1e-3 + 2.0 ** -8 * np.abs(ref)
        assert np.all(np.abs(got - ref) <= lim), f"delta check layer {l} proj {p}"
        worst = max(worst, err / tol)
    assert len(refs) == 32 * 7
    log(f"[parity] merged full stack worst err/tol {worst:.3f}")


# ---------------------------------------------------------- random cases ----
def multi_proj_case(seed, dtype="bf16", has_base=False, T=None, r_max=64):
    g = np.random.default_rng(seed)
    base = random_case(seed, dtype=dtype, has_base=has_base, T=T, r_max=r_max,
                       h_in=int(g.integers(1, 70)) * 8)
    nproj = int(g.integers(1, 4))
    projs = tuple(Proj(f"p{i}", base.projs[0].h_in, int(g.integers(1, 50)) * 8, "x")
                  for i in range(nproj))
    return dataclasses.replace(base, projs=projs, calls=(tuple(range(nproj)),))


@pytest.mark.parametrize("seed", range(16))
def test_random_heterogeneous(seed):
    dtype = "f32" if seed % 4 == 3 else "bf16"
    w = multi_proj_case(seed, dtype=dtype, has_base=seed % 2 == 0)
    log(f"[parity] random {seed} T={w.num_tokens} S={w.num_segs} projs="
        f"{[(p.h_in, p.h_out) for p in w.projs]} ranks={list(w.ranks)} {dtype}")
    dw = DeviceWorkload(w, threads=4)
    dw.run_fused()
    torch.cuda.synchronize()
    check_workload(dw, tight=True, threads=4)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("r_top", [4, 8, 16, 32, 64])
def test_decode_rank_bound(dtype, r_top):
    """Decode batches whose largest rank is r_top: the decode expand is built
    per bound on the B row width of the launch's rank classes, so each bound
    (and the classes below it in one launch) is checked."""
    seed = 200 + r_top + (1 if dtype == "f32" else 0)
    w = random_case(seed, T=48, h_in=264, h_out=200, n_adapters=6, max_seg=3,
                    r_choices=sorted({r_top, max(1, r_top // 2), max(1, r_top // 4), 1}),
                    dtype=dtype, has_base=r_top % 16 == 0)
    # adapter 0 has rank r_top and the first non-empty segment
    first = int(np.flatnonzero(np.diff(w.seg_starts) > 0)[0])
    w = dataclasses.replace(w, ranks=np.where(np.arange(w.pool_size) == 0, r_top, w.ranks)
                            .astype(np.int32), seg_adapter=np.where(
                                np.arange(w.num_segs) == first, 0, w.seg_adapter).astype(np.int32))
    log(f"[parity] decode rank bound {r_top} {dtype} ranks={list(w.ranks)}")
    dw = DeviceWorkload(w, threads=4)
    assert dw.plan.stats()["max_block_tokens"] <= 4
    dw.run_fused()
    torch.cuda.synchronize()
    check_workload(dw, tight=True, threads=4)


@pytest.mark.parametrize("seed", range(6))
def test_prefill_blocks(seed):
    """Long same-adapter segments (over 1024 tokens in long groups, so the
    prefill kernel runs): several 64-token blocks per group, ragged tails;
    launches of few tiles split each tile's output rows over 4 and 2
    workgroups (T up to 1601, and 2600), or not at all (4100)."""
    T = [1030, 1100, 1300, 1601, 2600, 4100][seed]
    w = random_case(100 + seed, T=T, h_in=512, h_out=256, n_adapters=3, max_seg=T,
                    no_adapter_frac=0.0, r_choices=[8, 16, 32, 64])
    log(f"[parity] prefill {seed} T={T} segments={list(np.diff(w.seg_starts))}")
    dw = DeviceWorkload(w, threads=4)
    assert dw.plan.stats()["max_block_tokens"] > 4
    dw.run_fused()
    torch.cuda.synchronize()
    check_workload(dw, tight=True, threads=4)


@pytest.mark.parametrize("nproj,dtype", [(2, "bf16"), (3, "bf16"), (2, "f32"), (3, "f32")])
def test_prefill_multi_projection(nproj, dtype):
    """Calls of 2 and 3 projections over blocks of several token tiles: the
    prefill kernel forms every projection's v from one load of x per K-block
    and expands each; ranks up to 64 (4 rank tiles), distinct h_out per
    projection, ragged prompts beside decode steps."""
    seed = {2: 91, 3: 92}[nproj] + (10 if dtype == "f32" else 0)
    base = mixed_case(seed, dtype=dtype, has_base=nproj == 3, h_in=520, h_out=8)
    g = np.random.default_rng(seed)
    projs = tuple(Proj(f"p{i}", 520, int(g.integers(4, 40)) * 8, "x") for i in range(nproj))
    w = dataclasses.replace(base, projs=projs, calls=(tuple(range(nproj)),))
    log(f"[parity] prefill {nproj} projections {dtype} T={w.num_tokens} "
        f"h_out={[p.h_out for p in projs]} ranks={sorted(set(w.ranks.tolist()))}")
    dw = DeviceWorkload(w, threads=4)
    assert dw.plan.stats()["max_block_tokens"] > 16
    dw.run_fused()
    torch.cuda.synchronize()
    check_workload(dw, tight=True, threads=4)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("has_base", [True, False])
def test_mixed_blocks(dtype, has_base):
    """Prompts and decode steps in one batch: the long groups take 64-token
    blocks (the prefill kernel), the short groups and the tokens without an
    adapter 4-token blocks (shrink and decode expand): three launches a call."""
    seed = {("bf16", True): 81, ("bf16", False): 82, ("f32", True): 83, ("f32", False): 84}[
        (dtype, has_base)]
    w = mixed_case(seed, dtype=dtype, has_base=has_base, h_in=384, h_out=264)
    sizes = np.diff(w.seg_starts)
    log(f"[parity] mixed {w.name} {dtype} base {has_base} T={w.num_tokens} S={w.num_segs}")
    dw = DeviceWorkload(w, threads=4)
    st = dw.plan.stats()
    assert st["max_block_tokens"] > 4 and (sizes[w.seg_adapter >= 0] <= 3).any()
    dw.run_fused()
    torch.cuda.synchronize()
    check_workload(dw, tight=True, threads=4)


@pytest.mark.parametrize("case,opts", [
    ("decode", dict(long_group=1, long_batch=1)),
    ("decode", dict(shrink_groups=16)),
    ("decode", dict(shrink_groups=4096)),
    ("mixed", dict(long_group=200, long_batch=1)),
    ("mixed", dict(long_group=1, long_batch=1, prefill_groups=1)),
    ("mixed", dict(prefill_groups=65536, shrink_groups=384)),
])
def test_plan_opts_parity(case, opts):
    """Plans built under other plan options (groups moved between the decode
    cut and the prompt kernel, other k-chunkings and row splits) give the
    delta within the float32 bound of the oracle."""
    if case == "decode":
        w = random_case(95, T=200, h_in=1024, h_out=520, n_adapters=40, max_seg=6,
                        r_choices=[8, 16, 32, 64], has_base=True)
    else:
        w = mixed_case(96, h_in=384, h_out=264, r_choices=[8, 16, 24, 64])
    log(f"[parity] plan options {case} {opts} T={w.num_tokens} S={w.num_segs}")
    dw = DeviceWorkload(w, threads=4, plan_opts=opts)
    assert {k: dw.plan.opts()[k] for k in opts} == opts
    dw.zero_outputs()
    dw.run_fused()
    torch.cuda.synchronize()
    check_workload(dw, tight=True, threads=4)


@pytest.mark.parametrize("kind,dtype,opts", [
    ("sigma-full", "bf16", dict(long_group=1, long_batch=1)),
    ("sigma-diag", "f32", dict(long_group=1, long_batch=1, prefill_groups=1)),
    ("sigma-full", "f32", dict(shrink_groups=4096)),
    ("merge", "bf16", dict(long_group=1, long_batch=1)),
    ("merge", "f32", dict(shrink_groups=7, prefill_groups=1)),
])
def test_plan_opts_other_plans(kind, dtype, opts):
    """Jointly compressed and merge plans under other plan options (every
    group through the prompt kernel, other k-chunkings and row splits): the
    same checks as their own parity tests."""
    if kind == "merge":
        test_merge_parity(dtype, False, 3, plan_opts=opts)
    else:
        test_sigma_parity(kind.split("-")[1], dtype, False, plan_opts=opts)


def test_two_step_path():
    """sgmv_shrink + sgmv_expand through a caller's v buffer: within the
    float32 bound of the oracle, deterministic, and bit-identical to
    sgmv_fused on both the decode path (every kernel sums the k-chunk
    partials in one order) and the prefill path (the prefill kernel's A step
    and B step alone form v and y as its fused form does), also over all
    three projections of a call."""
    three = dataclasses.replace(
        mixed_case(72, h_in=264, h_out=8, has_base=False),
        projs=tuple(Proj(f"p{i}", 264, ho, "x") for i, ho in enumerate((96, 40, 136))),
        calls=((0, 1, 2),))
    for w in (config(1), multi_proj_case(3, has_base=True), config(0),
              mixed_case(71, h_in=512, h_out=256, r_choices=[8, 24, 64]), three):
        log(f"[parity] two-step {w.name}")
        dw = DeviceWorkload(w, threads=4)
        outs = []
        for _ in range(2):
            dw.zero_outputs()
            dw.run_two_step()
            torch.cuda.synchronize()
            outs.append({k: from_device(v) for k, v in dw.y.items()})
        for k in outs[0]:
            assert np.array_equal(outs[0][k], outs[1][k]), k
        check_workload(dw, tight=True, threads=4)
        dw.zero_outputs()
        dw.run_fused()
        torch.cuda.synchronize()
        for k, v in dw.y.items():
            assert np.array_equal(from_device(v).view(np.uint8), outs[0][k].view(np.uint8)), k


@pytest.mark.parametrize("prefill", [False, True])
def test_shrink_output_layout(prefill):
    """v holds A x in columns [i*r_max, i*r_max + rank) and zeros up to r_max;
    rows of tokens without an adapter are left as they were.  Decode blocks
    (shrink and reduce) and a batch with long groups (the prefill kernel's A
    step) over three projections."""
    import heterogeneous_adapter_batching_amd as hab
    if prefill:
        base = mixed_case(74, h_in=264, h_out=8, r_choices=(8, 16, 24, 32), r_max=32)
        w = dataclasses.replace(
            base, projs=tuple(Proj(f"p{i}", 264, ho, "x") for i, ho in enumerate((96, 40, 136))),
            calls=((0, 1, 2),))
    else:
        w = multi_proj_case(7, T=40, r_max=32)
    w = dataclasses.replace(w, ranks=np.minimum(w.ranks, 32))
    dw = DeviceWorkload(w, threads=4)
    assert (dw.plan.stats()["max_block_tokens"] > 16) == prefill
    n = len(w.projs)
    v = torch.full((w.num_tokens, n * 32 + 8), 7.0, device="cuda")
    hab.sgmv_shrink(dw.pool, dw.plan, 0, tuple(range(n)), dw.x[(0, "x")], v)
    v = v.cpu().numpy()
    x = w.activation(0, "x").astype(np.float64)
    tok = w.token_adapter()
    for t in range(w.num_tokens):
        i = int(tok[t])
        if i < 0:
            assert np.all(v[t] == 7.0)
            continue
        for p in range(n):
            a, _ = w.adapter_block(i, 0, p)
            r = a.shape[0]
            ref = a.astype(np.float64) @ x[t]
            tol = 1e-5 * (np.abs(a) @ np.abs(x[t])) + 1e-30
            assert np.all(np.abs(v[t, p * 32:p * 32 + r] - ref) <= tol)
            assert np.all(v[t, p * 32 + r:(p + 1) * 32] == 0)
        assert np.all(v[t, n * 32:] == 7.0)


# ------------------------------------------------------------ exact pins ----
def test_b_zero_identity_bitexact():
    w = multi_proj_case(11, has_base=True, T=50)
    over = {}
    for a in range(w.pool_size):
        for p in range(len(w.projs)):
            A, B = w.adapter_block(a, 0, p)
            over[(a, 0, p)] = (A, np.zeros_like(B))
    w = dataclasses.replace(w, overrides=over)
    dw = DeviceWorkload(w, threads=4)
    dw.run_fused()
    torch.cuda.synchronize()
    for p in range(len(w.projs)):
        assert np.array_equal(dw.output(0, p), w.base_out(0, p))


def test_indicator_gather_bitexact():
    """Indicator adapters make every delta an exact integer that encodes the
    adapter id: the GPU's gather and segment indexing must reproduce the
    segment table exactly."""
    T, h_in, h_out, pool = 300, 64, 32, 400
    g = np.random.default_rng(17)
    cuts = np.sort(g.choice(np.arange(1, T), 90, replace=False))
    starts = np.concatenate([[0], cuts, [T]]).astype(np.int32)
    segs = g.integers(-1, pool, len(starts) - 1).astype(np.int32)
    ranks = g.choice([1, 8, 16, 24, 64], pool).astype(np.int32)
    base = random_case(0, T=T, h_in=h_in, h_out=h_out)
    over = {}
    for i in range(pool):
        r = int(ranks[i])
        a = np.zeros((r, h_in), np.float32)
        a[0, 0] = 1.0
        b = np.zeros((h_out, r), np.float32)
        b[0, 0], b[1, 0] = i % 128, i // 128
        if r > 1:
            b[2:, 1:] = 0.5          # multiplies exact zeros of v
        over[(i, 0, 0)] = (a, b)
    w = dataclasses.replace(base, num_tokens=T, seg_starts=starts, seg_adapter=segs,
                            pool_size=pool, ranks=ranks,
                            scales=np.full(pool, 2.0, np.float32), overrides=over,
                            seed=77)
    x = w.activation(0, "x")
    x[:, 0] = 1.0
    w.activation = lambda layer, key, _x=x: _x      # noqa: E731  (instance override)
    dw = DeviceWorkload(w, threads=4)
    dw.zero_outputs()
    dw.run_fused()
    torch.cuda.synchronize()
    y = dw.output(0, 0)
    tok = w.token_adapter()
    for t in range(T):
        i = int(tok[t])
        if i < 0:
            assert np.all(y[t] == 0), t
        else:
            assert y[t, 0] == 2 * (i % 128) and y[t, 1] == 2 * (i // 128), (t, i, y[t, :2])
            assert np.all(y[t, 2:] == 0), t


def test_padding_invariance_bitexact():
    """An adapter stored at rank r equals the same adapter zero-padded to a
    larger rank, bit for bit."""
    w = random_case(31, T=70, h_in=256, h_out=128, n_adapters=4, r_choices=[3, 5, 12, 20],
                    no_adapter_frac=0.0)
    dw = DeviceWorkload(w, threads=4)
    dw.run_fused()
    small = dw.output(0, 0)
    over, ranks = {}, np.full(w.pool_size, 64, np.int32)
    for a in range(w.pool_size):
        A, B = w.adapter_block(a, 0, 0)
        r = A.shape[0]
        Ap = np.zeros((64, 256), np.float32)
        Ap[:r] = A
        Bp = np.zeros((128, 64), np.float32)
        Bp[:, :r] = B
        over[(a, 0, 0)] = (Ap, Bp)
    w2 = dataclasses.replace(w, ranks=ranks, overrides=over)
    dw2 = DeviceWorkload(w2, threads=4)
    dw2.run_fused()
    torch.cuda.synchronize()
    assert np.array_equal(dw2.output(0, 0), small)


def test_permutation_and_split_invariance_bitexact():
    w = random_case(41, T=120, h_in=384, h_out=200 // 8 * 8, n_adapters=5, max_seg=30,
                    r_choices=[8, 16, 32])
    dw = DeviceWorkload(w, threads=4)
    dw.run_fused()
    y = dw.output(0, 0)
    x = w.activation(0, "x")
    perm = np.random.default_rng(1).permutation(w.num_segs)
    rows, starts = [], [0]
    for si in perm:
        rows.extend(range(w.seg_starts[si], w.seg_starts[si + 1]))
        starts.append(starts[-1] + w.seg_starts[si + 1] - w.seg_starts[si])
    wp = dataclasses.replace(w, seg_starts=np.asarray(starts, np.int32),
                             seg_adapter=w.seg_adapter[perm])
    wp.activation = lambda layer, key: x[rows]      # noqa: E731
    dwp = DeviceWorkload(wp, threads=4)
    dwp.run_fused()
    assert np.array_equal(dwp.output(0, 0), y[rows])
    # split every segment in two
    s2, a2 = [0], []
    for si in range(w.num_segs):
        lo, hi = int(w.seg_starts[si]), int(w.seg_starts[si + 1])
        s2 += [(lo + hi) // 2, hi]
        a2 += [w.seg_adapter[si]] * 2
    ws = dataclasses.replace(w, seg_starts=np.asarray(s2, np.int32),
                             seg_adapter=np.asarray(a2, np.int32))
    dws = DeviceWorkload(ws, threads=4)
    dws.run_fused()
    torch.cuda.synchronize()
    assert np.array_equal(dws.output(0, 0), y)


def test_determinism():
    w = config(3)
    dw = DeviceWorkload(w)
    outs = []
    for _ in range(2):
        dw.zero_outputs()
        dw.run_fused()
        torch.cuda.synchronize()
        outs.append({k: from_device(v) for k, v in dw.y.items()})
    for k in outs[0]:
        assert np.array_equal(outs[0][k], outs[1][k])


# ------------------------------------------------------------ edge cases ----
def test_edge_cases():
    cases = [
        random_case(51, T=0, h_in=64, h_out=32),                               # empty batch
        random_case(52, T=1, h_in=64, h_out=32, no_adapter_frac=0.0),          # one token
        random_case(53, T=64, h_in=64, h_out=32, n_adapters=1, max_seg=64,
                    no_adapter_frac=0.0),                                      # one full block
        random_case(54, T=37, h_in=14336, h_out=64, n_adapters=2,
                    r_choices=[64]),                                           # long h_in, r_max
        random_case(55, T=20, h_in=4104, h_out=4104, n_adapters=3),            # ragged widths
        random_case(56, T=30, h_in=64, h_out=32, no_adapter_frac=1.0, has_base=True),
    ]
    for w in cases:
        log(f"[parity] edge {w.name} T={w.num_tokens} h_in={w.projs[0].h_in} "
            f"h_out={w.projs[0].h_out}")
        dw = DeviceWorkload(w, threads=4)
        dw.run_fused()
        torch.cuda.synchronize()
        check_workload(dw, tight=w.projs[0].h_in < 10000, threads=4)


def test_call_errors_enqueue_nothing():
    import heterogeneous_adapter_batching_amd as hab
    w = random_case(61, T=10, h_in=64, h_out=32)
    dw = DeviceWorkload(w, threads=2)
    x, y = dw.x[(0, "x")], dw.y[(0, 0)]
    plan2 = hab.Plan(dw.pool, w.num_tokens, w.seg_starts, w.seg_adapter)   # not uploaded
    with pytest.raises(hab.LoraError) as ei:
        hab.sgmv_fused(dw.pool, plan2, 0, (0,), (0,), x, y)
    assert ei.value.status == -9
    for args, code in (((1, (0,), (0,)), -1), ((0, (1,), (0,)), -1), ((0, (0,), (8,)), -1),
                       ((0, (0,), (4,)), -1)):
        with pytest.raises(hab.LoraError) as ei:
            hab.sgmv_fused(dw.pool, dw.plan, args[0], args[1], args[2], x, y)
        assert ei.value.status == code, args
    dw.pool.unregister(int(w.touched()[0]) if len(w.touched()) else 0)
    with pytest.raises(hab.LoraError) as ei:
        hab.sgmv_fused(dw.pool, dw.plan, 0, (0,), (0,), x, y)
    assert ei.value.status == -9


def test_graph_replay_matches_eager():
    """The fused step captured in a HIP graph gives the eager result on every
    replay, with eager work and synchronisation between replays (the kernels
    keep no state between calls and record no memset nodes: every workspace
    entry a call reads, the same call wrote before)."""
    w = multi_proj_case(5, has_base=True, T=90)
    dw = DeviceWorkload(w, threads=4)
    dw.run_fused()
    torch.cuda.synchronize()
    eager = {k: from_device(v) for k, v in dw.y.items()}
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=s):
        dw.run_fused()
    for rep in range(4):
        dw.zero_outputs()                  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in dw.y.items():
            assert np.array_equal(from_device(v), eager[k]), (rep, k)
        dw.run_fused()                     # and an eager call on the same workspace
        torch.cuda.synchronize()
        for k, v in dw.y.items():
            assert np.array_equal(from_device(v), eager[k]), (rep, k)


@pytest.mark.parametrize("T", [40, 700])
def test_plan_reupload_same_workspace(T):
    """Plans uploaded in turn into one workspace: every launch sees the plan
    uploaded before it.  The kernels read plan memory (descriptors, token
    rows) by scalar loads, as memory that no launch changes while it runs;
    a new upload between launches must still reach the next launch.  The
    second plan gives each segment the adapter of the segment before it;
    the third upload restores the first plan, whose output bits come back."""
    import heterogeneous_adapter_batching_amd as hab
    w1 = random_case(91, T=T, h_in=256, h_out=160, n_adapters=6, r_choices=[8, 16, 32])
    ids = np.asarray(w1.seg_adapter)
    w2 = dataclasses.replace(w1, seg_adapter=np.roll(ids, 1))
    assert not np.array_equal(ids, np.asarray(w2.seg_adapter))
    # the rotation can move an adapter off an empty segment: upload what either plan uses
    both = sorted(set(w1.touched().tolist()) | set(w2.touched().tolist()))
    dw = DeviceWorkload(w1, threads=2, upload=both)
    mp = dw.max_proj
    p1 = dw.plan
    p2 = hab.Plan(dw.pool, w2.num_tokens, w2.seg_starts, w2.seg_adapter)
    ws = torch.empty(max(p1.workspace_bytes(mp), p2.workspace_bytes(mp)), dtype=torch.uint8,
                     device="cuda")
    outs = []
    for i, (plan, w) in enumerate(((p1, w1), (p2, w2), (p1, w1))):
        plan.upload(mp, ws=ws)
        dw.plan, dw.w = plan, w
        dw.zero_outputs()
        dw.run_fused()
        torch.cuda.synchronize()
        for k, v in dw.y.items():
            bad = ~np.isfinite(from_device(v))
            assert not bad.any(), (f"upload {i}: {int(bad.sum())} non-finite outputs in {k}, "
                                   f"token rows {sorted(set(np.nonzero(bad)[0].tolist()))[:12]}")
        check_workload(dw, threads=2)
        outs.append({k: from_device(v) for k, v in dw.y.items()})
    for k in outs[0]:
        assert np.array_equal(outs[0][k], outs[2][k]), k
        assert not np.array_equal(outs[0][k], outs[1][k]), k


def test_workspace_owner_refuses_stale_plan():
    """A workspace holds the tables of the plan uploaded into it last: a call
    with a plan uploaded there before is refused (it would read the other
    plan's descriptors) until that plan is uploaded again."""
    import heterogeneous_adapter_batching_amd as hab
    w = random_case(93, T=50, h_in=128, h_out=64, n_adapters=4, r_choices=[8, 16])
    dw = DeviceWorkload(w, threads=2)
    mp = dw.max_proj
    p1 = dw.plan
    p2 = hab.Plan(dw.pool, w.num_tokens, w.seg_starts, np.roll(w.seg_adapter, 1))
    ws = torch.empty(dw.pool.workspace_bytes(w.num_tokens, w.num_segs, mp), dtype=torch.uint8,
                     device="cuda")
    p1.upload(mp, ws=ws)
    p2.upload(mp, ws=ws)
    with pytest.raises(hab.LoraError) as ei:
        dw.run_fused()
    assert ei.value.status == -9 and "another plan" in ei.value.message
    p1.upload(mp, ws=ws)
    dw.zero_outputs()
    dw.run_fused()
    torch.cuda.synchronize()
    check_workload(dw, threads=2)


def test_plan_rebuild_parity():
    """One plan rebuilt in place for batch after batch (decode steps, prompts,
    mixed; cores of the rebuilt plan kept plain) in one workspace sized once
    by lora_workspace_bytes, uploaded each time and checked against the
    oracle; the rebuilt plan's outputs equal a fresh plan's bit for bit."""
    import heterogeneous_adapter_batching_amd as hab
    base = random_case(94, T=1200, h_in=256, h_out=136, n_adapters=8, max_seg=300,
                       r_choices=[8, 16, 32, 64], has_base=True)
    dw = DeviceWorkload(base, threads=4, upload=np.arange(base.pool_size))
    mp = dw.max_proj
    ws = torch.empty(dw.pool.workspace_bytes(1200, 1200, mp), dtype=torch.uint8, device="cuda")
    plan = dw.plan
    g = np.random.default_rng(94)
    for step in range(6):
        T = [1200, 37, 1100, 1, 600, 256][step]
        cuts = np.unique(np.concatenate([[0, T], g.integers(0, T + 1, g.integers(1, 40))]))
        ids = g.integers(-1, base.pool_size, len(cuts) - 1).astype(np.int32)
        if step % 2 == 0:                            # a few long groups
            ids = (np.arange(len(cuts) - 1) % 3).astype(np.int32)
        w = dataclasses.replace(base, num_tokens=T, seg_starts=cuts.astype(np.int32),
                                seg_adapter=ids)
        plan.rebuild(T, w.seg_starts, w.seg_adapter)
        plan.upload(mp, ws=ws)
        sub = DeviceWorkload.__new__(DeviceWorkload)
        sub.__dict__.update(dw.__dict__)
        sub.w = w
        sub.plan = plan
        sub.x = {k: v[:T] for k, v in dw.x.items()}
        sub.base = {k: v[:T] for k, v in dw.base.items()}
        sub.y = {k: torch.zeros_like(v[:T]) for k, v in dw.base.items()}
        log(f"[parity] rebuild step {step}: T={T} S={w.num_segs} {plan.stats()}")
        sub.run_fused()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in sub.y.items()}
        check_workload(sub, threads=4)
        fresh = hab.Plan(dw.pool, T, w.seg_starts, w.seg_adapter).upload(mp)
        sub.plan = fresh
        for v in sub.y.values():
            v.zero_()
        sub.run_fused()
        torch.cuda.synchronize()
        for k in got:
            assert torch.equal(got[k].view(torch.int16), sub.y[k].view(torch.int16)), (step, k)


def test_register_from_device_matches_host():
    """lora_pool_register from device tensors (the pack kernels: A K-blocked,
    B in row slices of permuted vectors) writes the same extent bytes as
    uploads from host arrays, hence the same output bits; ranks of 1, 2, 5
    and 8 vectors a bf16 row, h_out 96 (a ragged B slice either way)."""
    import heterogeneous_adapter_batching_amd as hab
    from synth.device import to_device, host_weights
    for dtype, h_in in (("bf16", 200), ("f32", 72), ("bf16", 4096)):
        w = random_case(81, T=40, h_in=h_in, h_out=96, n_adapters=4, dtype=dtype,
                        r_choices=[5, 16, 40, 64])
        dw = DeviceWorkload(w, threads=2)
        dw.run_fused()
        ref = dw.output(0, 0)
        pool2 = hab.Pool(1, [h_in], [96], w.r_max, dtype, max_slots=8,
                         slab_bytes=dw.pool.slab.numel())
        pool2.slab.fill_(0xFF)                   # NaN everywhere the pack must overwrite
        for a in range(w.pool_size):
            A, B = w.adapter_block(a, 0, 0)
            pool2.register(a, int(w.ranks[a]), float(w.scales[a]),
                           [to_device(A, dtype)[None]], [to_device(B, dtype)[None]])
        es = 2 if dtype == "bf16" else 4
        span = 32 if dtype == "bf16" else 16
        for a in w.touched():
            q1, q2 = dw.pool.query(int(a)), pool2.query(int(a))
            n = q1["r_pad"] * es * (-(-h_in // span) * span + 96)   # less the 256-byte tail
            s1 = dw.pool.slab[q1["offset"]:q1["offset"] + n].cpu().numpy()
            s2 = pool2.slab[q2["offset"]:q2["offset"] + n].cpu().numpy()
            assert np.array_equal(s1, s2), (dtype, int(a))
        plan2 = hab.Plan(pool2, w.num_tokens, w.seg_starts, w.seg_adapter).upload(1)
        y2 = torch.zeros_like(dw.y[(0, 0)])
        hab.sgmv_fused(pool2, plan2, 0, (0,), (0,), dw.x[(0, "x")], y2)
        torch.cuda.synchronize()
        assert np.array_equal(from_device(y2), ref), dtype


# ------------------------------------------- jointly compressed adapters ----
def _jd_check(dw):
    """Contract tolerance per output tensor, and the delta alone (y - y_in)
    to a tolerance scaled by the delta plus the single rounding of y."""
    w = dw.w
    for l in dw.layers:
        for p in range(len(w.projs)):
            got = dw.output(l, p).astype(np.float64)
            ref = oracle_ref(w, l, p, acc="f64")
            contract_check(got, ref, f"{w.name} layer {l} proj {p}")
            y_in = w.base_out(l, p).astype(np.float64) if w.has_base else 0.0
            d_ref = ref - y_in
            ulp = 2.0 ** -8 if w.dtype == "bf16" else 2.0 ** -24
            lim = 1e-4 * np.abs(d_ref).max() + ulp * np.abs(ref) + 1e-30
            assert np.all(np.abs((got - y_in) - d_ref) <= lim), f"{w.name} delta {l} {p}"


@pytest.mark.parametrize("kind", ["full", "diag"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("prefill", [False, True])
def test_sigma_parity(kind, dtype, prefill, plan_opts=None):
    """The three steps A, Sigma, B ("Compress then Serve", rebuttal pseudocode
    of add_lora_slice_with_sigma) against the oracle: mixed basis ranks,
    segments without a core or an adapter, decode blocks or prefill blocks;
    the fused call and shrink + expand_sigma through v are bit-identical."""
    from synth import jd_case
    seed = {("full", "bf16"): 1, ("full", "f32"): 2, ("diag", "bf16"): 3,
            ("diag", "f32"): 4}[(kind, dtype)] + (10 if prefill else 0)
    w = jd_case(seed, kind=kind, dtype=dtype, T=1500 if prefill else 96,
                max_seg=500 if prefill else 3)
    log(f"[parity] {w.name} dtype {dtype} prefill {prefill} {plan_opts or ''}")
    dw = DeviceWorkload(w, threads=4, plan_opts=plan_opts)
    if plan_opts is None:
        assert (dw.plan.stats()["max_block_tokens"] > 4) == prefill
    dw.zero_outputs()
    dw.run_fused()
    torch.cuda.synchronize()
    _jd_check(dw)
    fused = {k: from_device(v) for k, v in dw.y.items()}
    dw.zero_outputs()
    dw.run_two_step()
    torch.cuda.synchronize()
    for k, v in dw.y.items():
        assert np.array_equal(from_device(v).view(np.uint8), fused[k].view(np.uint8)), k


def test_sigma_identity_equals_plain_bitexact():
    """Identity cores (full and diagonal) and a plan without cores all give
    the plain two-step delta with the shared basis, bit for bit."""
    import heterogeneous_adapter_batching_amd as hab
    from synth import jd_case
    for kind in ("full", "diag"):
        w = jd_case(21, kind=kind, T=80, max_seg=4)
        dw = DeviceWorkload(w, threads=4)
        if kind == "full":
            dw.sigma.copy_(torch.eye(w.r_max, device="cuda").expand_as(dw.sigma))
        else:
            dw.sigma.fill_(1.0)
        dw.zero_outputs()
        dw.run_fused()
        torch.cuda.synchronize()
        with_cores = {k: from_device(v) for k, v in dw.y.items()}
        plain = hab.Plan(dw.pool, w.num_tokens, w.seg_starts, w.seg_adapter)
        plain.upload(dw.max_proj)
        for l in dw.layers:
            for ci, c in enumerate(dw.calls):
                y = torch.zeros_like(dw.y[(l, ci)])
                hab.sgmv_fused(dw.pool, plain, l, c, dw.y_offsets[ci],
                               dw.x[(l, w.projs[c[0]].x_key)], y, dw.base.get((l, ci)))
                torch.cuda.synchronize()
                assert np.array_equal(from_device(y).view(np.uint8),
                                      with_cores[(l, ci)].view(np.uint8)), (kind, l, ci)


def test_sigma_call_errors():
    """A plan naming a core beyond the table, a bad kind, or a wrong table
    shape is refused before anything runs; y is untouched."""
    import heterogeneous_adapter_batching_amd as hab
    from synth import jd_case
    w = jd_case(22, kind="full", T=40, max_seg=4)
    dw = DeviceWorkload(w, threads=4)
    l, c = dw.layers[0], dw.calls[0]
    x = dw.x[(l, w.projs[c[0]].x_key)]
    y = dw.y[(l, 0)]
    y.fill_(3.0)
    small = dw.sigma[: int(w.seg_sigma.max())].contiguous()       # one core short
    with pytest.raises(hab.LoraError):
        hab.sgmv_fused_sigma(dw.pool, dw.plan, l, c, dw.y_offsets[0], x, small, "full", y)
    with pytest.raises(ValueError):
        hab.sgmv_fused_sigma(dw.pool, dw.plan, l, c, dw.y_offsets[0], x, dw.sigma, "lower", y)
    with pytest.raises(ValueError):
        hab.sgmv_fused_sigma(dw.pool, dw.plan, l, c, dw.y_offsets[0], x, dw.sigma[..., 0].contiguous(),
                             "full", y)
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())


# ----------------------------------------------------------- weighted merge ----
def _merge_setup(seed, *, K, dtype, T, max_seg, h_in=256, h_out=192, n_adapters=5,
                 plan_opts=None, r_choices=(8, 16, 32)):
    """A pool of n_adapters (mixed ranks) and K merge slots per segment: a
    plain random batch gives the segments; each slot draws its own adapters
    (or -1) and weights; plan_opts are set on the pool before the plan."""
    import heterogeneous_adapter_batching_amd as hab
    w = random_case(seed, T=T, h_in=h_in, h_out=h_out, n_adapters=n_adapters,
                    r_choices=list(r_choices), dtype=dtype, max_seg=max_seg, has_base=True,
                    r_max=max(r_choices))
    g = np.random.default_rng(seed)
    S = w.num_segs
    seg_ad = g.integers(-1, n_adapters, (S, K)).astype(np.int32)
    seg_ad[:, 0] = w.seg_adapter                            # slot 0: the batch's own draw
    seg_w = g.uniform(-1.0, 1.5, (S, K)).astype(np.float32)
    dw = DeviceWorkload(w, upload=np.arange(n_adapters), threads=4)
    if plan_opts:
        dw.pool.set_plan_opts(**plan_opts)
    plan = hab.Plan.merge(dw.pool, w.num_tokens, w.seg_starts, seg_ad, seg_w).upload(1)
    return w, dw, plan, seg_ad, seg_w


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("prefill", [False, True])
@pytest.mark.parametrize("K", [3, 4])
def test_merge_parity(dtype, prefill, K, plan_opts=None):
    """K adapters merged per request with weights, in one pass (one shrink
    over every (token, slot) row, one expand that sums the weighted deltas
    and rounds y once), against the oracle's merge: the contract tolerance,
    and the delta within the float32 accumulation bound plus a single
    rounding of y; the fused, static-scratch and split calls agree bit for
    bit."""
    import heterogeneous_adapter_batching_amd as hab
    seed = (31 if dtype == "bf16" else 32) + (10 if prefill else 0) + 100 * (K - 3)
    w, dw, plan, seg_ad, seg_w = _merge_setup(seed, K=K, dtype=dtype,
                                              T=1300 if prefill else 64,
                                              max_seg=400 if prefill else 3,
                                              plan_opts=plan_opts)
    log(f"[parity] merge {w.name} K={K} {dtype} prefill {prefill} {plan.stats()} "
        f"{plan_opts or ''}")
    if plan_opts is None:
        assert (plan.stats()["max_block_tokens"] > 4) == prefill
    _check_merge(w, dw, plan, seg_ad, seg_w, dtype)


def _check_merge(w, dw, plan, seg_ad, seg_w, dtype):
    """A merge plan's fused call against the oracle's merge (the contract
    tolerance, and the delta within the float32 accumulation bound plus one
    rounding of y); the static-scratch and split calls give the same bits."""
    import heterogeneous_adapter_batching_amd as hab
    x = dw.x[(0, "x")]
    y = torch.zeros_like(dw.y[(0, 0)])
    hab.sgmv_fused(dw.pool, plan, 0, (0,), [0], x, y, dw.base[(0, 0)])
    torch.cuda.synchronize()
    adapters = {}
    for a in range(w.pool_size):
        A, B = w.adapter_block(a, 0, 0)
        adapters[a] = (A, B, float(w.scales[a]))
    y_in = w.base_out(0, 0)
    ref = oracle.lora_delta_merge(w.activation(0, "x"), w.seg_starts, seg_ad, seg_w, adapters,
                                  y_in, acc="f64", threads=4)
    got = from_device(y).astype(np.float64)
    contract_check(got, ref, f"merge {w.name}")
    ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -24
    d_ref = ref - y_in
    lim = 1e-4 * np.abs(d_ref).max() + ulp * np.abs(ref) + 1e-30
    err = np.abs(got - ref)
    assert np.all(err <= lim), float((err / lim).max())
    # the same bits from the other entry points
    y2 = torch.zeros_like(y)
    hab.sgmv_fused_static(dw.pool, plan, 0, (0,), [0], x, y2, dw.base[(0, 0)])
    y3 = torch.zeros_like(y)
    hab.sgmv_shrink_partials(dw.pool, plan, 0, (0,), x)
    hab.sgmv_expand_partials(dw.pool, plan, 0, (0,), [0], y3, dw.base[(0, 0)])
    torch.cuda.synchronize()
    for other in (y2, y3):
        assert np.array_equal(from_device(y).view(np.uint8), from_device(other).view(np.uint8))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("K", [2, 3])
def test_merge_decode_parity(dtype, K):
    """Decode merges: every segment one token (or empty), so every merge
    block holds one token and the merge expand runs its single-token build;
    ranks 8-64 (B rows of 1-8 vectors in bf16, 2-16 in float32) against the
    oracle's merge at the bounds of the merge parity test, and the three
    entry points bit for bit."""
    seed = (61 if dtype == "bf16" else 62) + 10 * K
    w, dw, plan, seg_ad, seg_w = _merge_setup(seed, K=K, dtype=dtype, T=150, max_seg=1,
                                              n_adapters=8, r_choices=(8, 16, 32, 64))
    lens = np.diff(np.asarray(w.seg_starts))
    assert lens.max() == 1 and (lens == 1).sum() > 100
    log(f"[parity] decode merge {w.name} K={K} {dtype} {plan.stats()}")
    _check_merge(w, dw, plan, seg_ad, seg_w, dtype)


def test_merge_one_slot_equals_plain_bitexact():
    """A decode batch merged from one slot of weight 1 gives the plain plan's
    output bit for bit (the merge expand forms the same float32 sums); with
    base and without (y accumulated in place)."""
    import heterogeneous_adapter_batching_amd as hab
    for has_base in (True, False):
        w = random_case(57 + has_base, T=90, h_in=264, h_out=200, n_adapters=5,
                        r_choices=[8, 16, 32, 64], has_base=has_base, max_seg=3)
        dw = DeviceWorkload(w, threads=4)
        merge = hab.Plan.merge(dw.pool, w.num_tokens, w.seg_starts, w.seg_adapter[:, None],
                               np.ones((w.num_segs, 1), np.float32)).upload(1)
        x = dw.x[(0, "x")]
        y1 = torch.randn(dw.y[(0, 0)].shape, device="cuda").to(dw.y[(0, 0)].dtype)
        y2 = y1.clone()
        hab.sgmv_fused(dw.pool, dw.plan, 0, (0,), [0], x, y1, dw.base.get((0, 0)))
        hab.sgmv_fused(dw.pool, merge, 0, (0,), [0], x, y2, dw.base.get((0, 0)))
        torch.cuda.synchronize()
        assert np.array_equal(from_device(y1).view(np.uint8), from_device(y2).view(np.uint8))


def test_merge_refused_calls():
    """The calls through a caller's v and the core calls refuse a merge plan."""
    import heterogeneous_adapter_batching_amd as hab
    w, dw, plan, seg_ad, seg_w = _merge_setup(58, K=2, dtype="bf16", T=20, max_seg=3)
    x = dw.x[(0, "x")]
    v = torch.zeros((w.num_tokens, w.r_max), dtype=torch.float32, device="cuda")
    y = torch.zeros_like(dw.y[(0, 0)])
    with pytest.raises(hab.LoraError):
        hab.sgmv_shrink(dw.pool, plan, 0, (0,), x, v)
    with pytest.raises(hab.LoraError):
        hab.sgmv_expand(dw.pool, plan, 0, (0,), [0], v, y)


def test_weight_one_equals_plain_bitexact():
    """A weighted plan with every weight 1 gives the plain plan's output bit
    for bit (decode and prefill blocks)."""
    import heterogeneous_adapter_batching_amd as hab
    for seed, T, max_seg in ((51, 120, 3), (52, 1300, 400)):
        w = random_case(seed, T=T, h_in=256, h_out=128, n_adapters=4, r_choices=[16, 32],
                        has_base=True, max_seg=max_seg, r_max=32)
        dw = DeviceWorkload(w, threads=4)
        ones = hab.Plan(dw.pool, w.num_tokens, w.seg_starts, w.seg_adapter,
                        seg_weight=np.ones(w.num_segs, np.float32))
        ones.upload(1)
        x = dw.x[(0, "x")]
        y1 = torch.zeros_like(dw.y[(0, 0)])
        y2 = torch.zeros_like(dw.y[(0, 0)])
        hab.sgmv_fused(dw.pool, dw.plan, 0, (0,), [0], x, y1, dw.base[(0, 0)])
        hab.sgmv_fused(dw.pool, ones, 0, (0,), [0], x, y2, dw.base[(0, 0)])
        torch.cuda.synchronize()
        assert np.array_equal(from_device(y1).view(np.uint8), from_device(y2).view(np.uint8))


def test_weight_errors():
    """A weight that is not finite is refused when the plan is built."""
    import heterogeneous_adapter_batching_amd as hab
    w = random_case(53, T=20, h_in=64, h_out=32)
    dw = DeviceWorkload(w, threads=4)
    bad = np.ones(w.num_segs, np.float32)
    bad[-1] = np.inf
    with pytest.raises(hab.LoraError):
        hab.Plan(dw.pool, w.num_tokens, w.seg_starts, w.seg_adapter, seg_weight=bad)


def test_split_fused_bitexact():
    """sgmv_shrink_partials then sgmv_expand_partials give sgmv_fused's bits
    (decode blocks, prefill blocks, a mixed batch; with and without base);
    the expand refuses partials of another call, and, for a plan with long
    groups, a workspace whose last shrink was the fused call's (whose long
    groups' v never left the prefill kernel)."""
    import heterogeneous_adapter_batching_amd as hab
    cases = (random_case(61, T=100, h_in=384, h_out=256, n_adapters=6, has_base=True, max_seg=3),
             random_case(62, T=1300, h_in=256, h_out=128, n_adapters=3, max_seg=600,
                         no_adapter_frac=0.0),
             mixed_case(63, h_in=256, h_out=192, has_base=False))
    for w in cases:
        log(f"[parity] split {w.name}")
        dw = DeviceWorkload(w, threads=4)
        x = dw.x[(0, "x")]
        base = dw.base.get((0, 0))
        y1 = torch.zeros_like(dw.y[(0, 0)])
        y2 = torch.zeros_like(dw.y[(0, 0)])
        hab.sgmv_fused(dw.pool, dw.plan, 0, (0,), [0], x, y1, base)
        if dw.plan.stats()["max_block_tokens"] > 16:
            with pytest.raises(hab.LoraError) as ei:
                hab.sgmv_expand_partials(dw.pool, dw.plan, 0, (0,), [0], y2, base)
            assert ei.value.status == -9
        hab.sgmv_shrink_partials(dw.pool, dw.plan, 0, (0,), x)
        hab.sgmv_expand_partials(dw.pool, dw.plan, 0, (0,), [0], y2, base)
        torch.cuda.synchronize()
        assert np.array_equal(from_device(y1).view(np.uint8), from_device(y2).view(np.uint8))
    with pytest.raises(hab.LoraError) as ei:     # partials of layer 0, expand of layer 1
        w = random_case(64, T=20, h_in=64, h_out=32)
        w = dataclasses.replace(w, num_layers=2)
        dw = DeviceWorkload(w, threads=4)
        hab.sgmv_shrink_partials(dw.pool, dw.plan, 0, (0,), dw.x[(0, "x")])
        hab.sgmv_expand_partials(dw.pool, dw.plan, 1, (0,), [0], dw.y[(1, 0)])
    assert ei.value.status == -9


@pytest.mark.parametrize("kind", ["full", "diag"])
def test_split_fused_sigma_bitexact(kind):
    """The split form with cores gives sgmv_fused_sigma's bits."""
    import heterogeneous_adapter_batching_amd as hab
    from synth import jd_case
    w = jd_case(71 if kind == "full" else 72, kind=kind, T=96, max_seg=3)
    log(f"[parity] split sigma {w.name}")
    dw = DeviceWorkload(w, threads=4)
    c = dw.calls[0]
    x = dw.x[(0, w.projs[c[0]].x_key)]
    base = dw.base.get((0, 0))
    y1 = torch.zeros_like(dw.y[(0, 0)])
    y2 = torch.zeros_like(dw.y[(0, 0)])
    hab.sgmv_fused_sigma(dw.pool, dw.plan, 0, c, dw.y_offsets[0], x, dw.sigma, kind, y1, base)
    hab.sgmv_shrink_partials(dw.pool, dw.plan, 0, c, x)
    hab.sgmv_expand_partials_sigma(dw.pool, dw.plan, 0, c, dw.y_offsets[0], dw.sigma, kind, y2,
                                   base)
    torch.cuda.synchronize()
    assert np.array_equal(from_device(y1).view(np.uint8), from_device(y2).view(np.uint8))
