"""Adapter exchange on the GPU: packed images, the residency cache's LRU
policy against a model of it, and the delta over a sequence of batches whose
adapters come and go while earlier batches still run, against the oracle."""
import dataclasses
import sys

import numpy as np
import pytest

import oracle
from synth import Proj, Workload
from synth.device import from_device, host_weights, to_device

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


def exchange_case(dtype, *, n_adapters=10, ranks=None, T=48, seed=0):
    """Two layers, two projections sharing x; adapters of the given ranks."""
    ranks = np.full(n_adapters, 16, np.int32) if ranks is None else np.asarray(ranks, np.int32)
    g = np.random.default_rng(seed)
    return Workload(
        name=f"exchange_{dtype}_{seed}", seed=4000 + seed, dtype=dtype, num_layers=2,
        projs=(Proj("q", 256, 192, "x"), Proj("k", 256, 64, "x")), calls=((0, 1),),
        num_tokens=T, seg_starts=np.arange(T + 1, dtype=np.int32),
        seg_adapter=np.zeros(T, np.int32), pool_size=len(ranks), ranks=ranks,
        scales=g.uniform(0.5, 2.0, len(ranks)).astype(np.float32), has_base=True, r_max=32,
        description="adapter exchange case")


def host_image(hab, desc, w, aid):
    """The adapter's packed extent image in pinned host memory."""
    r = int(w.ranks[aid])
    A = [np.stack([host_weights(w.adapter_block(aid, l, p)[0], w.dtype)
                   for l in range(w.num_layers)]) for p in range(len(w.projs))]
    B = [np.stack([host_weights(w.adapter_block(aid, l, p)[1], w.dtype)
                   for l in range(w.num_layers)]) for p in range(len(w.projs))]
    img = torch.empty(hab.extent_bytes(desc, r), dtype=torch.uint8, pin_memory=True)
    hab.pack_adapter(desc, r, A, B, out=img.numpy())
    return img


def batch_segments(g, T, ids_pool, k):
    """A batch of T tokens in segments naming k distinct adapters of
    ids_pool (and some tokens without an adapter)."""
    chosen = g.choice(ids_pool, k, replace=False)
    cuts = np.sort(g.choice(np.arange(1, T), 2 * k - 1, replace=False))
    starts = np.concatenate([[0], cuts, [T]]).astype(np.int32)
    segs = np.asarray([chosen[i % k] for i in range(2 * k)], np.int32)
    segs[g.random(2 * k) < 0.1] = -1
    return starts, segs


class LruModel:
    """The cache policy for adapters of one size in a pool of `cap` of them:
    misses in first-appearance order; a full pool evicts the resident adapter
    with the oldest use, ties to the lowest id, never one of the batch."""

    def __init__(self, cap):
        self.cap, self.tick, self.res = cap, 0, {}
        self.hits = self.misses = self.prefetched = self.evictions = 0

    def _bring(self, a, keep):
        if len(self.res) == self.cap:
            cand = [(t, i) for i, t in self.res.items() if i not in keep]
            if not cand:
                return False
            self.res.pop(min(cand)[1])
            self.evictions += 1
        self.res[a] = self.tick
        return True

    def acquire(self, ids):
        self.tick += 1
        order = list(dict.fromkeys(int(i) for i in ids if i >= 0))
        for a in order:
            if a in self.res:
                self.hits += 1
            else:
                assert self._bring(a, set(order))
                self.misses += 1
            self.res[a] = self.tick

    def prefetch(self, ids, held=()):
        """held: the outstanding batch's adapters, which are never evicted."""
        self.tick += 1
        keep = set()
        for a in (int(i) for i in ids):
            if a < 0 or a in keep:
                continue
            keep.add(a)
            if a in self.res:
                self.res[a] = self.tick
                continue
            if not self._bring(a, keep | set(held)):
                break
            self.prefetched += 1


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_register_image_matches_register(dtype):
    """An adapter copied as one packed image fills its extent exactly as the
    per-block upload does (padded ranks, ragged K-blocks)."""
    import heterogeneous_adapter_batching_amd as hab
    w = dataclasses.replace(exchange_case(dtype, ranks=[5, 16, 24]),
                            projs=(Proj("q", 200, 72, "x"), Proj("k", 200, 16, "x")))
    pools = [hab.Pool(w.num_layers, [p.h_in for p in w.projs], [p.h_out for p in w.projs],
                      w.r_max, dtype, slab_bytes=sum(
                          hab.extent_bytes(hab.api.make_desc(
                              w.num_layers, [p.h_in for p in w.projs],
                              [p.h_out for p in w.projs], w.r_max, dtype), int(r))
                          for r in w.ranks)) for _ in range(2)]
    for pl in pools:
        pl.slab.fill_(0x5A)
    imgs = []
    for a in range(w.pool_size):
        r = int(w.ranks[a])
        A = [np.stack([host_weights(w.adapter_block(a, l, p)[0], dtype)
                       for l in range(w.num_layers)]) for p in range(len(w.projs))]
        B = [np.stack([host_weights(w.adapter_block(a, l, p)[1], dtype)
                       for l in range(w.num_layers)]) for p in range(len(w.projs))]
        pools[0].register(a, r, float(w.scales[a]), A, B)
        imgs.append(host_image(hab, pools[1].desc, w, a))
        pools[1].register_image(a, r, float(w.scales[a]), imgs[-1])
    torch.cuda.synchronize()
    es = 2 if dtype == "bf16" else 4
    span = 32 if dtype == "bf16" else 16
    row = sum(-(-p.h_in // span) * span + p.h_out for p in w.projs)
    for a in range(w.pool_size):
        q0, q1 = pools[0].query(a), pools[1].query(a)
        n = q0["r_pad"] * es * w.num_layers * row          # the extent less its 256-byte tail
        s0 = pools[0].slab[q0["offset"]:q0["offset"] + n].cpu().numpy()
        s1 = pools[1].slab[q1["offset"]:q1["offset"] + n].cpu().numpy()
        assert np.array_equal(s0, s1), a


def _run_batches(hab, w, cache, pool, batches, *, prefetch_next=False, model=None):
    """Every batch on one compute stream with no host wait between batches:
    acquire, plan, the fused delta of each layer into its own output, release
    (then, optionally, prefetch the next batch's adapters)."""
    comp = torch.cuda.Stream()
    x = {l: to_device(w.activation(l, "x"), w.dtype) for l in range(w.num_layers)}
    base = {l: to_device(np.concatenate([w.base_out(l, p) for p in range(2)], axis=1), w.dtype)
            for l in range(w.num_layers)}
    outs, plans, ups = [], [], []
    torch.cuda.synchronize()
    with torch.cuda.stream(comp):
        for bi, (starts, segs) in enumerate(batches):
            ups.append(cache.acquire(segs, stream=comp))
            if model:
                model.acquire(segs)
            if prefetch_next and bi + 1 < len(batches):     # copies under this batch
                cache.prefetch(batches[bi + 1][1])
                if model:
                    model.prefetch(batches[bi + 1][1], held=set(int(i) for i in segs if i >= 0))
            plan = hab.Plan(pool, w.num_tokens, starts, segs)
            plan.upload(2, stream=comp)
            ys = {}
            for l in range(w.num_layers):
                ys[l] = torch.empty((w.num_tokens, 256), device="cuda",
                                    dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32)
                hab.sgmv_fused(pool, plan, l, (0, 1), [0, 192], x[l], ys[l], base[l], stream=comp)
            cache.release(stream=comp)
            outs.append(ys)
            plans.append(plan)
    torch.cuda.synchronize()
    return outs, ups


def _check_batches(w, batches, outs):
    for bi, (starts, segs) in enumerate(batches):
        wb = dataclasses.replace(w, seg_starts=starts, seg_adapter=segs)
        for l in range(w.num_layers):
            got = from_device(outs[bi][l])
            for p, (o0, o1) in enumerate(((0, 192), (192, 256))):
                ref = oracle.workload_call(wb, l, p, acc="f64", threads=4)
                tol = 1e-2 * float(np.abs(ref).max()) + 1e-3
                err = float(np.abs(got[:, o0:o1] - ref).max())
                assert err <= tol, f"batch {bi} layer {l} proj {p}: {err:.3e} > {tol:.3e}"


@pytest.mark.parametrize("dtype,prefetch", [("bf16", False), ("bf16", True), ("f32", False)])
def test_cache_lru_sequence(dtype, prefetch):
    """12 batches of 3 adapters each over 10 adapters in a pool that holds 4:
    hits, misses, prefetches and evictions follow the LRU model exactly, and
    every batch's delta matches the oracle although copies for later batches
    are enqueued while earlier ones still run."""
    import heterogeneous_adapter_batching_amd as hab
    w = exchange_case(dtype, seed=1 if prefetch else 0)
    desc = hab.api.make_desc(w.num_layers, [p.h_in for p in w.projs],
                             [p.h_out for p in w.projs], w.r_max, dtype)
    ext = hab.extent_bytes(desc, 16)
    pool = hab.Pool(w.num_layers, [p.h_in for p in w.projs], [p.h_out for p in w.projs],
                    w.r_max, dtype, slab_bytes=4 * ext)
    cache = hab.Cache(pool)
    for a in range(w.pool_size):
        cache.add(a, 16, float(w.scales[a]), host_image(hab, desc, w, a))
    g = np.random.default_rng(7 + prefetch)
    batches = [batch_segments(g, w.num_tokens, np.arange(w.pool_size), 3) for _ in range(12)]
    log(f"[exchange] {dtype} prefetch {prefetch}: "
        f"{[sorted(set(s[s >= 0].tolist())) for _, s in batches]}")
    model = LruModel(4)
    outs, ups = _run_batches(hab, w, cache, pool, batches, prefetch_next=prefetch, model=model)
    st = cache.stats()
    assert (st["hits"], st["misses"], st["prefetched"], st["evictions"]) == (
        model.hits, model.misses, model.prefetched, model.evictions), (st, vars(model))
    assert st["resident"] == len(model.res) and st["bytes_uploaded"] == ext * (
        model.misses + model.prefetched)
    for a in range(w.pool_size):
        assert cache.query(a) == {"resident": a in model.res, "held": False}
    if prefetch:
        assert st["prefetched"] > 0
    _check_batches(w, batches, outs)


def test_cache_mixed_ranks():
    """Adapters of ranks 8..32 in a slab that fits about half of them:
    evictions free extents of other sizes; deltas match the oracle.  (The
    slab holds three of the largest extents, so that a batch of two always
    fits however the first of them splits the free space.)"""
    import heterogeneous_adapter_batching_amd as hab
    g = np.random.default_rng(3)
    w = exchange_case("bf16", ranks=g.choice([8, 16, 24, 32], 12), seed=2)
    desc = hab.api.make_desc(w.num_layers, [p.h_in for p in w.projs],
                             [p.h_out for p in w.projs], w.r_max, "bf16")
    total = sum(hab.extent_bytes(desc, int(r)) for r in w.ranks)
    pool = hab.Pool(w.num_layers, [p.h_in for p in w.projs], [p.h_out for p in w.projs],
                    w.r_max, "bf16",
                    slab_bytes=max(total // 2 // 256 * 256, 3 * hab.extent_bytes(desc, 32)))
    cache = hab.Cache(pool)
    for a in range(w.pool_size):
        cache.add(a, int(w.ranks[a]), float(w.scales[a]), host_image(hab, desc, w, a))
    batches = [batch_segments(g, w.num_tokens, np.arange(w.pool_size), 2) for _ in range(10)]
    outs, _ = _run_batches(hab, w, cache, pool, batches, prefetch_next=True)
    st = cache.stats()
    log(f"[exchange] mixed ranks: {st}")
    assert st["evictions"] > 0
    _check_batches(w, batches, outs)


def test_cache_errors_and_stale_plan():
    import heterogeneous_adapter_batching_amd as hab
    w = exchange_case("bf16", n_adapters=4, seed=3)
    desc = hab.api.make_desc(w.num_layers, [p.h_in for p in w.projs],
                             [p.h_out for p in w.projs], w.r_max, "bf16")
    ext = hab.extent_bytes(desc, 16)
    pool = hab.Pool(w.num_layers, [p.h_in for p in w.projs], [p.h_out for p in w.projs],
                    w.r_max, "bf16", slab_bytes=2 * ext)
    cache = hab.Cache(pool)
    imgs = [host_image(hab, desc, w, a) for a in range(4)]
    for a in range(3):
        cache.add(a, 16, 1.0, imgs[a])

    def status(fn, *args):
        with pytest.raises(hab.LoraError) as ei:
            fn(*args)
        return ei.value.status

    assert status(cache.add, 0, 16, 1.0, imgs[0]) == -8          # added already
    pool.register_image(3, 16, 1.0, imgs[3])
    torch.cuda.synchronize()
    assert status(cache.add, 3, 16, 1.0, imgs[3]) == -8          # in the pool by other means
    pool.unregister(3)
    assert status(cache.acquire, [7]) == -3                      # not added
    assert status(cache.release) == -9                           # nothing outstanding
    assert status(cache.acquire, [0, 1, 2]) == -2                # 3 do not fit in 2
    assert cache.acquire([0, 1]) == 0                            # both resident already
    assert status(cache.acquire, [0]) == -9                      # one outstanding already
    cache.release()
    starts, segs = np.array([0, 10, 20], np.int32), np.array([0, 1], np.int32)
    old = hab.Plan(pool, 20, starts, segs)
    old.upload(2)
    assert cache.acquire([2, -1]) == 1                           # evicts adapter 0
    cache.release()
    x = to_device(w.activation(0, "x")[:20], "bf16")
    y = torch.zeros((20, 256), device="cuda", dtype=torch.bfloat16)
    assert status(hab.sgmv_fused, pool, old, 0, (0, 1), [0, 192], x, y) == -9
    torch.cuda.synchronize()
    assert cache.query(0) == {"resident": False, "held": False}
    assert cache.query(2) == {"resident": True, "held": False}
