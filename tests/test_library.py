"""Host-side tests of the C-ABI library (no GPU calls).

- every function include/lora_sgmv.h declares is exported by libhab_lora.so;
- the pool's byte accounting reproduces the adapter size the pages print
  ("TGI Multi-LoRA: Deploy Once, Serve 30 Models", "Technical Foundation":
  13.6 MB adapter, 14.48 GB Mistral-7B base, under a thousandth, 30 adapters
  about 3% of VRAM);
- validation rejects malformed input with the documented status and leaves
  the pool unchanged;
- the gather plan (first-appearance grouping, token order, blocks) is
  bit-exact against an independent re-implementation.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import heterogeneous_adapter_batching_amd as hab
from heterogeneous_adapter_batching_amd.api import make_desc
from synth import mixed_case, random_case, config
from conftest import ROOT, read_golden

HEADER = os.path.join(ROOT, "include", "lora_sgmv.h")
MISTRAL = dict(h=4096, kv=1024, ffn=14336, layers=32)


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_header_symbols_exported():
    names = header_functions()
    assert len(names) >= 18, names
    from heterogeneous_adapter_batching_amd import build
    for path in (hab.LIB_PATH, build.DEBUG_LIB):
        lib = ctypes.CDLL(path)
        missing = [n for n in names if not hasattr(lib, n)]
        assert not missing, (path, missing)
    # and the binding declares every one of them
    from heterogeneous_adapter_batching_amd._lib import SIGNATURES
    assert sorted(SIGNATURES) == names


def test_debug_checks_flag():
    """lora_debug_checks: the release build reports no checks and no errors
    without touching a device; the debug build reports its checks (asked for
    the flag alone, it touches no device either)."""
    from heterogeneous_adapter_batching_amd import build
    assert hab.debug_checks() == (False, 0)
    assert hab.debug_checks(clear=True) == (False, 0)
    dbg = ctypes.CDLL(build.DEBUG_LIB)
    dbg.lora_debug_checks.argtypes = [ctypes.POINTER(ctypes.c_int32),
                                      ctypes.POINTER(ctypes.c_uint32), ctypes.c_int32]
    en = ctypes.c_int32(-1)
    assert dbg.lora_debug_checks(ctypes.byref(en), None, 0) == 0
    assert en.value == 1
    rel = hab.load()
    en = ctypes.c_int32(-1)
    assert rel.lora_debug_checks(ctypes.byref(en), None, 1) == 0 and en.value == 0


def _pool(**kw):
    args = dict(num_layers=1, h_in=[64], h_out=[32], r_max=64, dtype="bf16",
                slab_ptr=1 << 20, slab_bytes=1 << 24)
    args.update(kw)
    return hab.Pool(**args)


def test_pages_adapter_size():
    fig = {k: float(v[0]) for k, v in read_golden("pages_figures.txt")}
    h, kv, L = MISTRAL["h"], MISTRAL["kv"], MISTRAL["layers"]
    # three readings of the 13.6 MB adapter, all exactly 13,631,488 bytes
    readings = [
        (make_desc(L, [h, h], [h, kv], 16, "bf16"), 16),          # q, v at r=16, 16-bit
        (make_desc(L, [h, h], [h, kv], 8, "f32"), 8),             # q, v at r=8, fp32
        (make_desc(L, [h, h, h, h], [h, kv, kv, h], 8, "bf16"), 8),  # q, k, v, o at r=8
    ]
    base = fig["base_gb"] * 1e9
    for d, r in readings:
        b = hab.pool_bytes_for(d, r)
        assert b == 13_631_488
        assert round(b / 1e6, 1) == fig["adapter_mb"]
        assert b / base < fig["adapter_base_ratio_max"]
        pct = fig["adapters_loaded"] * b / base * 100
        assert round(pct) == fig["vram_increase_pct"]          # 2.8% -> "roughly 3%"
        assert hab.extent_bytes(d, r) == b                      # no padding at these ranks
    # the full-stack workload's adapter: 7 projections, r=16, bf16
    w = config(4)
    d = make_desc(32, [p.h_in for p in w.projs], [p.h_out for p in w.projs], 16, "bf16")
    assert hab.pool_bytes_for(d, 16) == 83_886_080


def test_extent_padding_and_alignment():
    d = make_desc(2, [64, 128], [32, 16], 64, "bf16", rank_granule=8)
    per_rank = 2 * 2 * (64 + 32 + 128 + 16)      # bytes per rank row over layers, projections
    assert hab.pool_bytes_for(d, 5) == 5 * per_rank
    assert hab.extent_bytes(d, 5) == -(-8 * per_rank // 256) * 256
    assert hab.extent_bytes(d, 65) == 0 and hab.pool_bytes_for(d, 0) == 0
    d16 = make_desc(2, [64, 128], [32, 16], 64, "bf16", rank_granule=16)
    assert hab.extent_bytes(d16, 5) == -(-16 * per_rank // 256) * 256


def test_pool_allocator_reuse_and_coalesce():
    d = make_desc(1, [64], [32], 64, "bf16")
    e8 = hab.extent_bytes(d, 8)
    pool = _pool(slab_bytes=4 * e8)
    for i in range(4):
        pool.reserve(i, 8, 1.0)
    with pytest.raises(hab.LoraError) as ei:
        pool.reserve(9, 8, 1.0)
    assert ei.value.status == -2                                   # ENOSPC
    pool.unregister(1)
    pool.unregister(2)                                             # coalesce 1+2
    pool.reserve(10, 16, 1.0)                                      # needs 2 * e8
    assert pool.query(10)["offset"] == e8
    assert pool.stats() == {"adapters": 3, "free_bytes": 0}


def test_pool_validation_leaves_state():
    pool = _pool(max_slots=2)
    pool.reserve(1, 8, 2.0)
    before = pool.stats()
    cases = [((1, 8, 1.0), -8), ((2, 0, 1.0), -4), ((2, 65, 1.0), -4), ((-3, 8, 1.0), -1)]
    for args, code in cases:
        with pytest.raises(hab.LoraError) as ei:
            pool.reserve(*args)
        assert ei.value.status == code, args
        assert pool.stats() == before
    pool.reserve(2, 8, 1.0)
    with pytest.raises(hab.LoraError) as ei:
        pool.reserve(3, 8, 1.0)
    assert ei.value.status == -2                                   # slots full
    with pytest.raises(hab.LoraError) as ei:
        pool.unregister(7)
    assert ei.value.status == -3
    with pytest.raises(hab.LoraError) as ei:
        pool.query(7)
    assert ei.value.status == -3


def test_bad_descriptors():
    for kw, code in (({"h_in": [60]}, -1), ({"r_max": 12}, -1), ({"r_max": 128}, -1),
                     ({"dtype": "bf16", "rank_granule": 4}, -1)):
        with pytest.raises(hab.LoraError) as ei:
            _pool(**kw)
        assert ei.value.status == code, kw


def test_segment_validation():
    pool = _pool()
    pool.reserve(4, 8, 1.0)
    bad = [
        (5, [1, 5], [4], -6),            # does not start at 0
        (5, [0, 4], [4], -6),            # does not end at T
        (5, [0, 3, 2, 5], [4, 4, 4], -6),  # decreasing
        (5, [0, 5], [6], -3),            # unknown id
        (5, [0, 5], [-2], -3),           # ids below -1
        (-1, [0], [], -6),
    ]
    for T, starts, segs, code in bad:
        with pytest.raises(hab.LoraError) as ei:
            hab.Plan(pool, T, starts, segs)
        assert ei.value.status == code, (T, starts, segs)
    # empty batch, empty segments, only "no adapter" tokens: all valid
    assert hab.Plan(pool, 0, [0], []).stats()["groups"] == 0
    assert hab.Plan(pool, 3, [0, 0, 3, 3], [4, -1, 4]).stats() == {
        "groups": 0, "blocks": 1, "active_tokens": 0, "max_block_tokens": 3}


def reference_plan(T, starts, segs, ranks):
    """Independent re-implementation of the gather: groups in order of first
    appearance among non-empty segments, each group's tokens in segment order,
    then every token without an adapter in ascending order."""
    order_ids, members = [], {}
    for s in range(len(segs)):
        a = int(segs[s])
        if a < 0 or starts[s + 1] == starts[s]:
            continue
        if a not in members:
            order_ids.append(a)
            members[a] = []
        members[a].extend(range(starts[s], starts[s + 1]))
    tok_group = np.full(T, -1, np.int32)
    order = []
    for g, a in enumerate(order_ids):
        order.extend(members[a])
        tok_group[members[a]] = g
    order.extend(t for t in range(T) if tok_group[t] < 0)
    return (np.asarray(order, np.int32), tok_group, np.asarray(order_ids, np.int32),
            np.asarray([ranks[a] for a in order_ids], np.int32))


@pytest.mark.parametrize("seed", range(16))
def test_plan_matches_reference(seed):
    if seed < 10:
        w = random_case(seed, T=int(np.random.default_rng(seed).integers(0, 300)),
                        h_in=64, h_out=32)
    elif seed < 13:                     # long groups, some holding 1024 tokens between them
        w = random_case(seed, T=int(np.random.default_rng(seed).integers(900, 2500)),
                        h_in=64, h_out=32, n_adapters=4)
    else:                               # prompts and decode steps in one batch
        w = mixed_case(seed, h_in=64, h_out=32, long_tokens=1000 + 40 * seed)
    pool = _pool(max_slots=w.pool_size)
    for i in range(w.pool_size):
        pool.reserve(i, int(w.ranks[i]), float(w.scales[i]))
    plan = hab.Plan(pool, w.num_tokens, w.seg_starts, w.seg_adapter)
    got = plan.export()
    ref = reference_plan(w.num_tokens, w.seg_starts, w.seg_adapter, w.ranks)
    for k, r in zip(("token_order", "token_group", "group_adapter", "group_rank"), ref):
        assert np.array_equal(got[k], r), k
    st = plan.stats()
    assert st["active_tokens"] == int((ref[1] >= 0).sum())
    check_blocks(st, ref)


def _cut(n, m):
    k = -(-n // m)
    return [n // k + (i < n % k) for i in range(k)]


def check_blocks(st, ref, long_group=48, long_batch=1024):
    """The plan's block counts from the reference grouping: shrink blocks are
    near-equal cuts of each group into at most 16 tokens, each cut again into
    near-equal expand blocks of at most 4 tokens; both levels 64 tokens for a
    group of >= long_group tokens, once such groups hold >= long_batch tokens
    between them."""
    sizes = np.bincount(ref[1][ref[1] >= 0], minlength=len(ref[2]))
    use_long = sizes[sizes >= long_group].sum() >= long_batch

    def n_expand_blocks(n, long):
        smax, emax = (64, 64) if long else (16, 4)
        return sum(len(_cut(sn, emax)) for sn in _cut(n, smax)) if n else 0

    exp_blocks = sum(n_expand_blocks(int(n), use_long and n >= long_group) for n in sizes) + \
        n_expand_blocks(int((ref[1] < 0).sum()), False)
    long_sizes = sizes[sizes >= long_group] if use_long else sizes[:0]
    assert st["max_block_tokens"] <= (64 if use_long else 4)
    assert (st["max_block_tokens"] > 4) == bool(use_long and (long_sizes > 4).any())
    assert st["blocks"] == exp_blocks


def test_plan_opts_defaults_and_validation():
    """lora_plan_opts: the defaults, a pool's options set and read back, and
    out-of-range values refused with LORA_EINVAL, the pool's options then
    unchanged."""
    assert hab.plan_opts_default() == dict(long_group=48, long_batch=1024, shrink_groups=128,
                                           prefill_groups=256)
    pool = _pool()
    assert pool.plan_opts() == hab.plan_opts_default()
    pool.set_plan_opts(long_group=5, long_batch=7, shrink_groups=384, prefill_groups=65536)
    want = dict(long_group=5, long_batch=7, shrink_groups=384, prefill_groups=65536)
    assert pool.plan_opts() == want
    for bad in (dict(long_group=0), dict(long_batch=-3), dict(shrink_groups=0),
                dict(shrink_groups=65537), dict(prefill_groups=0), dict(prefill_groups=1 << 20)):
        with pytest.raises(hab.LoraError) as ei:
            pool.set_plan_opts(**bad)
        assert ei.value.status == -1, bad
        assert pool.plan_opts() == want
    lib = hab.load()
    o = hab.PlanOpts()
    assert lib.lora_pool_set_plan_opts(None, ctypes.byref(o)) == -1
    assert lib.lora_pool_set_plan_opts(pool.handle, None) == -1
    assert lib.lora_pool_get_plan_opts(pool.handle, None) == -1
    assert lib.lora_plan_get_opts(None, ctypes.byref(o)) == -1
    with pytest.raises(ValueError):
        pool.set_plan_opts(tile_tokens=8)


@pytest.mark.parametrize("long_group,long_batch", [(1, 1), (3, 40), (48, 1024), (200, 1)])
def test_plan_opts_grouping(long_group, long_batch):
    """A plan cuts its groups by the long-group thresholds of the options it
    was built with (the pool's when it was built), against the reference."""
    for seed in (3, 11, 14):
        if seed < 10:
            w = random_case(seed, T=250, h_in=64, h_out=32)
        elif seed < 13:
            w = random_case(seed, T=1500, h_in=64, h_out=32, n_adapters=4)
        else:
            w = mixed_case(seed, h_in=64, h_out=32, long_tokens=1200)
        pool = _pool(max_slots=w.pool_size)
        for i in range(w.pool_size):
            pool.reserve(i, int(w.ranks[i]), float(w.scales[i]))
        pool.set_plan_opts(long_group=long_group, long_batch=long_batch)
        plan = hab.Plan(pool, w.num_tokens, w.seg_starts, w.seg_adapter)
        assert plan.opts()["long_group"] == long_group
        ref = reference_plan(w.num_tokens, w.seg_starts, w.seg_adapter, w.ranks)
        got = plan.export()
        for k, r in zip(("token_order", "token_group", "group_adapter", "group_rank"), ref):
            assert np.array_equal(got[k], r), k
        check_blocks(plan.stats(), ref, long_group, long_batch)
        # the plan keeps its options when the pool's change; a rebuild takes
        # the pool's new ones
        before = (plan.stats(), plan.workspace_bytes(3))
        pool.set_plan_opts(long_group=48, long_batch=1024, shrink_groups=1024)
        assert (plan.stats(), plan.workspace_bytes(3)) == before
        assert plan.opts()["long_group"] == long_group
        plan.rebuild(w.num_tokens, w.seg_starts, w.seg_adapter)
        assert plan.opts() == pool.plan_opts()
        check_blocks(plan.stats(), ref)


def test_plan_for_workloads():
    """Groups of the five workloads' segment tables (the gather each launch does)."""
    expect_groups = {0: None, 1: None, 2: 8, 3: None, 4: None}
    for i in range(5):
        w = config(i)
        pool = hab.Pool(w.num_layers, [p.h_in for p in w.projs], [p.h_out for p in w.projs],
                        w.r_max, w.dtype, max_slots=w.pool_size, slab_ptr=1 << 20,
                        slab_bytes=1 << 40)
        for a in range(w.pool_size):
            pool.reserve(a, int(w.ranks[a]), float(w.scales[a]))
        plan = hab.Plan(pool, w.num_tokens, w.seg_starts, w.seg_adapter)
        st = plan.stats()
        assert st["groups"] == len(w.touched())
        if expect_groups[i] is not None:
            assert st["groups"] == expect_groups[i]
        assert st["active_tokens"] == w.num_tokens


def _b_block(b, dtype):
    """B [h_out][r_pad] (pads included) in the header's B layout: rows in
    slices of 64 * rpl, each slice's 16-byte vectors ordered (i, v, l) for
    row base + rpl * l + i, vector v; built by index arithmetic on a
    [slice rows][vectors][elements] view."""
    h_out, r_pad = b.shape
    per = 8 if dtype == "bf16" else 4                    # elements of a 16-byte vector
    nv = r_pad // per
    nvt = 1 << (nv - 1).bit_length()
    rpl = 1 if nvt >= 8 else 2
    out = []
    for base in range(0, h_out, 64 * rpl):
        n = min(64 * rpl, h_out - base)
        sl = b[base:base + n].reshape(n // rpl, rpl, nv, per)   # [l][i][v][e]
        out.append(sl.transpose(1, 2, 0, 3).ravel())            # [i][v][l][e]
    return np.concatenate(out)


def _pack_reference(L, h_in, h_out, rank, r_pad, span, dtype):
    """The extent image as the header lays it out, built with numpy: per layer
    (outermost) and projection, A K-blocked [h_in_pad / span][r_pad][span],
    then the B block (_b_block); pads zero; the whole rounded up to 256
    bytes."""
    g = np.random.default_rng(rank * 7 + len(h_in))
    npdt = np.uint16 if dtype == "bf16" else np.float32
    A = [g.integers(1, 60000, (L, rank, hi)).astype(npdt) if dtype == "bf16"
         else g.standard_normal((L, rank, hi)).astype(npdt) for hi in h_in]
    B = [g.integers(1, 60000, (L, ho, rank)).astype(npdt) if dtype == "bf16"
         else g.standard_normal((L, ho, rank)).astype(npdt) for ho in h_out]
    parts = []
    for l in range(L):
        for p, (hi, ho) in enumerate(zip(h_in, h_out)):
            hp = -(-hi // span) * span
            a = np.zeros((r_pad, hp), npdt)
            a[:rank, :hi] = A[p][l]
            parts.append(a.reshape(r_pad, hp // span, span).transpose(1, 0, 2).ravel())
            b = np.zeros((ho, r_pad), npdt)
            b[:, :rank] = B[p][l]
            parts.append(_b_block(b, dtype))
    raw = np.concatenate(parts).view(np.uint8)
    img = np.zeros(-(-raw.size // 256) * 256, np.uint8)
    img[:raw.size] = raw
    return A, B, img


@pytest.mark.parametrize("dtype,rank,granule", [("bf16", 5, 8), ("bf16", 16, 16),
                                                 ("bf16", 27, 8), ("bf16", 64, 8),
                                                 ("f32", 13, 8), ("f32", 32, 8)])
def test_pack_adapter_layout(dtype, rank, granule):
    """lora_pack_adapter writes the extent layout the header states, byte for
    byte, with ragged h_in (not a multiple of the K-block), padded ranks and
    B blocks of one, several and ragged row slices (rows of 1 to 8 vectors:
    two rows a lane and one)."""
    h_in, h_out, L = [40, 96, 24], [24, 8, 328], 3
    desc = make_desc(L, h_in, h_out, 64, dtype, rank_granule=granule)
    r_pad = -(-rank // granule) * granule
    span = 32 if dtype == "bf16" else 16
    A, B, ref = _pack_reference(L, h_in, h_out, rank, r_pad, span, dtype)
    assert hab.extent_bytes(desc, rank) == ref.size
    got = hab.pack_adapter(desc, rank, A, B)
    assert np.array_equal(got, ref)
    # a dirty output buffer is overwritten everywhere, tail included
    out = np.full(ref.size + 64, 0xAB, np.uint8)
    hab.pack_adapter(desc, rank, A, B, out=out)
    assert np.array_equal(out[:ref.size], ref) and (out[ref.size:] == 0xAB).all()


def test_pack_adapter_errors():
    desc = make_desc(1, [16], [16], 16, "f32")
    A, B = [np.zeros((1, 4, 16), np.float32)], [np.zeros((1, 16, 4), np.float32)]
    with pytest.raises(hab.LoraError) as ei:
        hab.pack_adapter(desc, 4, A, B, out=np.zeros(8, np.uint8))
    assert ei.value.status == -1
    with pytest.raises(hab.LoraError) as ei:
        hab.pack_adapter(desc, 17, A, B)
    assert ei.value.status == -4


def _random_plans(n):
    """Random batches over small pools of mixed ranks: decode-like, prompt-like
    (long groups holding 1024 tokens and more) and mixed."""
    for seed in range(n):
        g = np.random.default_rng(700 + seed)
        kind = seed % 3
        if kind == 0:
            w = random_case(700 + seed, T=int(g.integers(0, 400)), h_in=64, h_out=32)
        elif kind == 1:
            w = random_case(700 + seed, T=int(g.integers(1000, 3000)), h_in=64, h_out=32,
                            n_adapters=int(g.integers(1, 5)))
        else:
            w = mixed_case(700 + seed, h_in=64, h_out=32, long_tokens=1000 + 10 * seed)
        yield w


@pytest.mark.parametrize("dtype,h_in,opts", [
    ("bf16", [64, 64, 4104], {}), ("f32", [64, 1000, 64], {}),
    ("bf16", [64, 64, 4104], dict(long_group=1, long_batch=1, shrink_groups=1024)),
    ("bf16", [4096, 64, 14336], dict(long_group=20, long_batch=100, shrink_groups=7)),
    ("f32", [64, 1000, 64], dict(long_batch=1, shrink_groups=65536))])
def test_workspace_bound(dtype, h_in, opts):
    """lora_workspace_bytes bounds the workspace of every plan of at most
    that many tokens and segments, for calls of 1..3 projections, under the
    pool's plan options."""
    for w in _random_plans(24 if not opts else 12):
        pool = hab.Pool(1, h_in, [32, 48, 16], 64, dtype, max_slots=w.pool_size,
                        slab_ptr=1 << 20, slab_bytes=1 << 30)
        pool.set_plan_opts(**opts)
        for i in range(w.pool_size):
            pool.reserve(i, int(w.ranks[i]), float(w.scales[i]))
        plan = hab.Plan(pool, w.num_tokens, w.seg_starts, w.seg_adapter)
        for mp in (1, 2, 3):
            need = plan.workspace_bytes(mp)
            bound = pool.workspace_bytes(w.num_tokens, w.num_segs, mp)
            assert 0 < need <= bound, (w.name, mp, need, bound)
    assert pool.workspace_bytes(-1, 1, 1) == 0 and pool.workspace_bytes(1, 1, 9) == 0


def test_plan_rebuild_matches_create():
    """A plan rebuilt in place for batch after batch holds what a new plan of
    the same batch holds; a rebuild that fails leaves the plan as it was."""
    pool = _pool(max_slots=64, h_in=[64], h_out=[32])
    g = np.random.default_rng(5)
    for i in range(64):
        pool.reserve(i, int(g.integers(1, 65)), float(g.uniform(0.5, 2)))
    plan = None
    for seed, w in enumerate(_random_plans(12)):
        ids = np.where(w.seg_adapter >= 0, w.seg_adapter % 64, -1).astype(np.int32)
        fresh = hab.Plan(pool, w.num_tokens, w.seg_starts, ids)
        if plan is None:
            plan = hab.Plan(pool, w.num_tokens, w.seg_starts, ids)
        else:
            plan.rebuild(w.num_tokens, w.seg_starts, ids)
        a, b = plan.export(), fresh.export()
        for k in a:
            assert np.array_equal(a[k], b[k]), (seed, k)
        assert plan.stats() == fresh.stats()
        assert plan.workspace_bytes(3) == fresh.workspace_bytes(3)
        before = (plan.export(), plan.stats())
        with pytest.raises(hab.LoraError) as ei:
            plan.rebuild(w.num_tokens + 1, w.seg_starts, ids)      # does not end at T
        assert ei.value.status == -6
        after = (plan.export(), plan.stats())
        assert after[1] == before[1]
        for k in before[0]:
            assert np.array_equal(after[0][k], before[0][k])
    # weights and cores through rebuild
    plan.rebuild(4, [0, 2, 4], [1, 2], seg_weight=[0.5, 2.0])
    plan.rebuild(4, [0, 2, 4], [1, 2], seg_sigma=[0, -1])
    with pytest.raises(hab.LoraError):
        plan.rebuild(4, [0, 2, 4], [1, 2], seg_weight=[np.inf, 2.0])


def test_merge_plan_validation():
    """lora_plan_create_merge: slot counts outside 1..LORA_MAX_MERGE, a bad
    segment table, an unknown slot adapter and a weight that is not finite
    are refused; a valid plan has a row per (token, non-empty slot), its
    workspace within the bound for that many rows, and no export."""
    pool = _pool(max_slots=8)
    for i in range(4):
        pool.reserve(i, 8 * (i + 1), 1.0)
    starts = [0, 3, 5]
    ads = np.array([[0, 1, -1], [2, 2, 3]], np.int32)
    wts = np.array([[1.0, 0.5, 2.0], [0.25, -1.0, 3.0]], np.float32)
    plan = hab.Plan.merge(pool, 5, starts, ads, wts)
    st = plan.stats()
    assert st["active_tokens"] == 3 * 2 + 2 * 3               # rows of non-empty slots
    assert st["groups"] == 4
    assert 0 < plan.workspace_bytes(1) <= pool.workspace_bytes(st["active_tokens"], 6, 1)
    with pytest.raises(hab.LoraError):
        plan.export()
    bad = [(np.zeros((2, 0), np.int32), np.zeros((2, 0), np.float32), -1),     # K = 0
           (np.zeros((2, 5), np.int32), np.ones((2, 5), np.float32), -1),      # K = 5
           (np.array([[0], [7]], np.int32), np.ones((2, 1), np.float32), -3),  # unknown id
           (np.array([[0], [1]], np.int32), np.array([[1.0], [np.nan]], np.float32), -1)]
    for a, w_, code in bad:
        with pytest.raises(hab.LoraError) as ei:
            hab.Plan.merge(pool, 5, starts, a, w_)
        assert ei.value.status == code, (a.shape, code)
    with pytest.raises(hab.LoraError) as ei:
        hab.Plan.merge(pool, 6, starts, ads, wts)               # does not end at T
    assert ei.value.status == -6
