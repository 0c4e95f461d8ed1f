"""Seeded synthetic workloads for the multi-adapter LoRA delta.

This module only draws inputs: token activations, segment tables, adapter
ranks, adapter weights and base outputs.  It holds none of the delta's
arithmetic, so both the CPU oracle and the GPU path can consume what it
produces without sharing any computation.

The five Mistral-7B-shaped workloads follow the shapes of the multi-LoRA
serving pages (a Mistral-7B base with one LoRA per request and a pool of
more than a thousand adapters: "Compress then Serve", reviews and
rebuttal; "TGI Multi-LoRA: Deploy Once, Serve 30 Models", "How Multi-LoRA
Serving Works").  Their trained adapters and datasets are not available, so
every value here is random with the stated distribution:

  x ~ N(0, 1), A ~ U(-1/sqrt(h_in), +1/sqrt(h_in)), B ~ N(0, 0.02^2),
  base_out ~ N(0, 1), scale = alpha / r with alpha = 2 r.

For bf16 workloads every value is rounded once, to nearest-even, to a
bf16-representable float32.  The float32 arrays returned here therefore hold
exactly the numbers the GPU receives as bf16 bit patterns.

Every block has its own seed (``numpy.random.SeedSequence`` over a tuple of
integers), so a test can regenerate one (adapter, layer, projection) block
without drawing the rest of an 84 GB pool.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import os

import numpy as np

# Tags that keep the per-block seed tuples of different kinds apart.
_TAG_MAP, _TAG_RANK, _TAG_W, _TAG_X, _TAG_BASE, _TAG_SIGMA = 1, 2, 7, 11, 13, 17


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); return float32.

    NaN payloads are kept quiet; inputs here are finite, so the plain
    integer rounding rule applies.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) & np.uint32(0xFFFF0000)).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The bf16 bit patterns (uint16) of float32 values that are bf16-exact."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("values are not bf16-representable")
    return (u >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


@dataclass(frozen=True)
class Proj:
    """One adapted linear layer: h_in -> h_out, fed by activation ``x_key``."""
    name: str
    h_in: int
    h_out: int
    x_key: str


@dataclass
class Workload:
    name: str
    seed: int
    dtype: str                      # "f32" or "bf16"
    num_layers: int
    projs: tuple                    # tuple[Proj, ...]
    calls: tuple                    # projection index tuples launched together
    num_tokens: int
    seg_starts: np.ndarray          # int32 [S+1]
    seg_adapter: np.ndarray         # int32 [S]
    pool_size: int
    ranks: np.ndarray               # int32 [pool_size]
    scales: np.ndarray              # float32 [pool_size]
    has_base: bool
    r_max: int = 64
    description: str = ""
    # Adapter weights drawn for a pin instead of the random recipe:
    # {(adapter, layer, proj): (A, B)}.
    overrides: dict = field(default_factory=dict)
    # Jointly compressed adapters: the pool entries are shared bases, and
    # segment s also names core seg_sigma[s] (-1: none) of n_cores cores of
    # kind sigma_kind ("full": r_max x r_max, "diag": r_max values).
    seg_sigma: np.ndarray = None
    n_cores: int = 0
    sigma_kind: str = None
    # Weighted merging: segment s merges the adapters merge_ids[s] (K slots,
    # -1: an empty slot) with weights merge_w[s]; seg_adapter is then slot 0.
    merge_ids: np.ndarray = None
    merge_w: np.ndarray = None

    # ---- derived facts about the draw (pure bookkeeping) ----
    @property
    def num_segs(self) -> int:
        return int(self.seg_adapter.shape[0])

    def token_adapter(self) -> np.ndarray:
        """Adapter id of every token row (the per-token ``indices`` form)."""
        ids = np.full(self.num_tokens, -1, dtype=np.int32)
        for s in range(self.num_segs):
            ids[self.seg_starts[s]:self.seg_starts[s + 1]] = self.seg_adapter[s]
        return ids

    def touched(self) -> np.ndarray:
        """Distinct adapter ids the batch uses (every merge slot included), in
        first-appearance order."""
        out, seen = [], set()
        for s in range(self.num_segs):
            slots = self.merge_ids[s] if self.merge_ids is not None else (self.seg_adapter[s],)
            for a in slots:
                a = int(a)
                if a >= 0 and self.seg_starts[s + 1] > self.seg_starts[s] and a not in seen:
                    seen.add(a)
                    out.append(a)
        return np.asarray(out, dtype=np.int32)

    def token_slots(self) -> np.ndarray:
        """Adapter ids of every token row's slots, [T][K] (K = 1 without
        merging; -1: none)."""
        ids = self.merge_ids if self.merge_ids is not None else self.seg_adapter[:, None]
        out = np.full((self.num_tokens, ids.shape[1]), -1, dtype=np.int32)
        for s in range(self.num_segs):
            out[self.seg_starts[s]:self.seg_starts[s + 1]] = ids[s]
        return out

    def x_keys(self) -> list:
        keys = []
        for p in self.projs:
            if p.x_key not in keys:
                keys.append(p.x_key)
        return keys

    def x_width(self, key: str) -> int:
        return next(p.h_in for p in self.projs if p.x_key == key)

    # ---- values ----
    def _round(self, a: np.ndarray) -> np.ndarray:
        return bf16_round(a) if self.dtype == "bf16" else a.astype(np.float32)

    def adapter_block(self, aid: int, layer: int, p: int):
        """(A [r][h_in], B [h_out][r]) float32 for one adapter, layer, projection."""
        key = (int(aid), int(layer), int(p))
        if key in self.overrides:
            a, b = self.overrides[key]
            return np.asarray(a, np.float32), np.asarray(b, np.float32)
        pr = self.projs[p]
        r = int(self.ranks[aid])
        g = _rng(self.seed, _TAG_W, aid, layer, p)
        bound = np.float32(1.0 / np.sqrt(pr.h_in))
        a = (g.random((r, pr.h_in), dtype=np.float32) * np.float32(2.0) - np.float32(1.0)) * bound
        b = g.standard_normal((pr.h_out, r), dtype=np.float32) * np.float32(0.02)
        return self._round(a), self._round(b)

    def core(self, j: int, layer: int, p: int) -> np.ndarray:
        """Core j of (layer, projection p), float32: full cores are the
        identity plus N(0, 1/r_max) noise, diagonal cores U(0.5, 1.5)."""
        g = _rng(self.seed, _TAG_SIGMA, j, layer, p)
        r = self.r_max
        if self.sigma_kind == "full":
            c = np.eye(r, dtype=np.float32) + g.standard_normal((r, r), dtype=np.float32) * \
                np.float32(1.0 / np.sqrt(r))
            return c.astype(np.float32)
        return (g.random(r, dtype=np.float32) + np.float32(0.5)).astype(np.float32)

    def core_table(self) -> np.ndarray:
        """All cores: [n_cores][layers][projections][r_max]([r_max])."""
        return np.stack([np.stack([np.stack([self.core(j, l, p) for p in range(len(self.projs))])
                                   for l in range(self.num_layers)])
                         for j in range(self.n_cores)])

    def activation(self, layer: int, key: str) -> np.ndarray:
        """x [T][h_in] float32 for the activation ``key`` of ``layer``."""
        k = self.x_keys().index(key)
        g = _rng(self.seed, _TAG_X, layer, k)
        x = g.standard_normal((self.num_tokens, self.x_width(key)), dtype=np.float32)
        return self._round(x)

    def base_out(self, layer: int, p: int) -> np.ndarray:
        """base_out [T][h_out] float32 (the frozen layer's W x, given)."""
        g = _rng(self.seed, _TAG_BASE, layer, p)
        y = g.standard_normal((self.num_tokens, self.projs[p].h_out), dtype=np.float32)
        return self._round(y)

    def adapter_full(self, aid: int, p: int, threads: int = 0):
        """(A [L][r][h_in], B [L][h_out][r]) for every layer of one adapter."""
        layers = range(self.num_layers)
        if threads and self.num_layers > 1:
            with ThreadPoolExecutor(threads) as ex:
                blocks = list(ex.map(lambda l: self.adapter_block(aid, l, p), layers))
        else:
            blocks = [self.adapter_block(aid, l, p) for l in layers]
        return (np.stack([b[0] for b in blocks]), np.stack([b[1] for b in blocks]))


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ---------------------------------------------------------------------------
# The five workloads (Mistral-7B shapes: hidden 4096, kv 1024, ffn 14336).
# ---------------------------------------------------------------------------
H, KV, FFN, LAYERS = 4096, 1024, 14336, 32
MISTRAL_PROJS = (
    Proj("q", H, H, "attn"), Proj("k", H, KV, "attn"), Proj("v", H, KV, "attn"),
    Proj("o", H, H, "o"), Proj("gate", H, FFN, "mlp"), Proj("up", H, FFN, "mlp"),
    Proj("down", FFN, H, "down"),
)


def _one_token_segments(T: int):
    return np.arange(T + 1, dtype=np.int32)


def config0() -> Workload:
    """Tiny fp32: h=256, 4 rank-8 adapters, 16 tokens in 4 segments of 4."""
    seed = 0
    ids = _rng(seed, _TAG_MAP).integers(0, 4, 4).astype(np.int32)
    return Workload(
        name="tiny_f32", seed=seed, dtype="f32", num_layers=1,
        projs=(Proj("p", 256, 256, "x"),), calls=((0,),), num_tokens=16,
        seg_starts=np.arange(0, 17, 4, dtype=np.int32), seg_adapter=ids,
        pool_size=4, ranks=np.full(4, 8, np.int32), scales=np.full(4, 2.0, np.float32),
        has_base=False, r_max=8,
        description="h_in=h_out=256, 4 adapters r=8 s=2, T=16 in 4 segments of 4, fp32")


def config1() -> Workload:
    """q_proj decode: 64 tokens, one per request, 32 rank-16 adapters."""
    seed = 1
    ids = _rng(seed, _TAG_MAP).integers(0, 32, 64).astype(np.int32)
    return Workload(
        name="q_decode_bf16", seed=seed, dtype="bf16", num_layers=1,
        projs=(Proj("q", H, H, "attn"),), calls=((0,),), num_tokens=64,
        seg_starts=_one_token_segments(64), seg_adapter=ids,
        pool_size=32, ranks=np.full(32, 16, np.int32), scales=np.full(32, 2.0, np.float32),
        has_base=False, r_max=16,
        description="q 4096->4096, T=S=64, 32 adapters r=16 s=2, ids uniform")


def config2() -> Workload:
    """Heterogeneous prefill: 8 requests x 512 tokens, q/k/v/o, rank 16."""
    seed = 2
    projs = (Proj("q", H, H, "attn"), Proj("k", H, KV, "attn"),
             Proj("v", H, KV, "attn"), Proj("o", H, H, "o"))
    return Workload(
        name="prefill_bf16", seed=seed, dtype="bf16", num_layers=1,
        projs=projs, calls=((0, 1, 2), (3,)), num_tokens=4096,
        seg_starts=np.arange(0, 4097, 512, dtype=np.int32),
        seg_adapter=np.arange(8, dtype=np.int32),
        pool_size=8, ranks=np.full(8, 16, np.int32), scales=np.full(8, 2.0, np.float32),
        has_base=False, r_max=16,
        description="q,o 4096->4096; k,v 4096->1024; T=4096 as 8 segments of 512; r=16")


def config3() -> Workload:
    """Multi-rank decode: 256 tokens over a pool of 1000, ranks {8,16,32,64}."""
    seed = 3
    ids = _rng(seed, _TAG_MAP).integers(0, 1000, 256).astype(np.int32)
    ranks = _rng(seed, _TAG_RANK).choice(np.array([8, 16, 32, 64]), 1000).astype(np.int32)
    projs = (Proj("gate", H, FFN, "mlp"), Proj("up", H, FFN, "mlp"),
             Proj("down", FFN, H, "down"))
    return Workload(
        name="multirank_decode_bf16", seed=seed, dtype="bf16", num_layers=1,
        projs=projs, calls=((0, 1), (2,)), num_tokens=256,
        seg_starts=_one_token_segments(256), seg_adapter=ids,
        pool_size=1000, ranks=ranks,
        scales=(2.0 * ranks / ranks).astype(np.float32),   # alpha / r with alpha = 2 r
        has_base=False, r_max=64,
        description="gate/up 4096->14336, down 14336->4096; T=S=256; pool 1000, r in {8,16,32,64}")


def zipf_probs(n: int, s: float) -> np.ndarray:
    """Bounded Zipf popularity: P(id = k) proportional to (k+1)^-s, k < n."""
    w = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    return w / w.sum()


def config4() -> Workload:
    """Full Mistral-7B LoRA stack: 32 layers x 7 projections, Zipf(1.1) decode."""
    seed = 4
    ids = _rng(seed, _TAG_MAP).choice(1000, size=128, p=zipf_probs(1000, 1.1)).astype(np.int32)
    return Workload(
        name="full_stack_bf16", seed=seed, dtype="bf16", num_layers=LAYERS,
        projs=MISTRAL_PROJS, calls=((0, 1, 2), (3,), (4, 5), (6,)), num_tokens=128,
        seg_starts=_one_token_segments(128), seg_adapter=ids,
        pool_size=1000, ranks=np.full(1000, 16, np.int32),
        scales=np.full(1000, 2.0, np.float32), has_base=True, r_max=16,
        description="32 layers x {q,k,v,o,gate,up,down}; T=S=128; pool 1000 r=16; "
                    "Zipf(1.1) popularity; y = base_out + delta")


def merge_full_stack(K: int = 2) -> Workload:
    """The full stack with every decode request merging K adapters: slot 0
    is the plain full stack's Zipf(1.1) draw, slots 1..K-1 independent draws
    of the same law, weights U(0.2, 1.0) per (request, slot)."""
    seed = 7
    w = config4()
    S = w.num_segs
    ids = np.empty((S, K), np.int32)
    ids[:, 0] = w.seg_adapter
    p = zipf_probs(1000, 1.1)
    for k in range(1, K):
        g = _rng(seed, _TAG_MAP, k)
        for s in range(S):                  # K distinct adapters a request
            a = int(g.choice(1000, p=p))
            while a in ids[s, :k]:
                a = int(g.choice(1000, p=p))
            ids[s, k] = a
    wts = (_rng(seed, _TAG_MAP, 100).random((S, K), dtype=np.float32) * np.float32(0.8) +
           np.float32(0.2)).astype(np.float32)
    w.name = f"full_stack_merge{K}_bf16"
    w.merge_ids, w.merge_w = ids, wts
    w.description = (f"32 layers x {{q,k,v,o,gate,up,down}}; T=S=128; pool 1000 r=16; "
                     f"each request merges {K} adapters (Zipf(1.1) draws, weights "
                     "U(0.2, 1)); y = base_out + sum_k w_k delta_k")
    return w


def sweep_stack(n_adapters: int = 128) -> Workload:
    """The full stack of the Zipf decode batch with a pool of n_adapters
    rank-16 adapters, every one of them used by the first draw (token t takes
    adapter t mod n_adapters).  Activations and base outputs are the same
    draws as the Zipf batch's; only the assignment differs."""
    w = config4()
    T = w.num_tokens
    w.name = "full_stack_sweep_bf16"
    w.pool_size = n_adapters
    w.ranks = np.full(n_adapters, 16, np.int32)
    w.scales = np.full(n_adapters, 2.0, np.float32)
    w.seg_adapter = (np.arange(T) % n_adapters).astype(np.int32)
    w.description = (f"32 layers x {{q,k,v,o,gate,up,down}}; T=S={T}; pool {n_adapters} r=16; "
                     "the assignment of tokens to adapters varies")
    return w


def sweep_assignments(T: int = 128, n_adapters: int = 128):
    """Token-to-adapter assignments of the cost sweep, as (label, params,
    ids[T]).  Adapter identity does not change the work, only how many
    distinct adapters there are and how many tokens each takes, so every
    draw is relabelled to ids 0, 1, ... in order of first appearance.

    * ``distinct``: d distinct adapters, token t takes t mod d (d = 0: no
      token is adapted); d runs over 0, 1, 2, 4, ..., T.
    * ``zipf``: T ids drawn from a bounded Zipf(s) over 1000 adapters, for a
      range of skews s (s = 0 is uniform)."""
    out = []
    d = 0
    while d <= min(T, n_adapters):
        ids = np.full(T, -1, np.int32) if d == 0 else (np.arange(T) % d).astype(np.int32)
        out.append((f"distinct={d}", {"kind": "distinct", "d": d}, ids))
        d = 1 if d == 0 else 2 * d
    for k, s in enumerate((0.0, 0.5, 0.8, 1.1, 1.5, 2.0, 3.0)):
        draw = _rng(4, _TAG_MAP, 1000 + k).choice(1000, size=T, p=zipf_probs(1000, s))
        relabel = {}
        ids = np.asarray([relabel.setdefault(int(a), len(relabel)) for a in draw], np.int32)
        assert len(relabel) <= n_adapters
        out.append((f"zipf={s}", {"kind": "zipf", "s": s}, ids))
    return out


CONFIGS = (config0, config1, config2, config3, config4)


def config(i: int) -> Workload:
    return CONFIGS[i]()


def random_case(seed: int, *, T: int = None, h_in: int = None, h_out: int = None,
                n_adapters: int = None, r_choices=None, dtype: str = "bf16",
                no_adapter_frac: float = 0.1, has_base: bool = False,
                max_seg: int = None, r_max: int = 64) -> Workload:
    """A small random heterogeneous batch: random segment cuts (empty segments
    included), repeated ids, id -1 (no adapter), mixed ranks 1..r_max and
    distinct random per-adapter scales."""
    g = _rng(seed, 99)
    T = int(g.integers(1, 65)) if T is None else T
    h_in = int(g.integers(1, 40)) * 8 if h_in is None else h_in
    h_out = int(g.integers(1, 40)) * 8 if h_out is None else h_out
    n_adapters = int(g.integers(1, 9)) if n_adapters is None else n_adapters
    cuts = [0]
    while cuts[-1] < T:
        step = int(g.integers(0, (max_seg or max(2, T // 3)) + 1))
        cuts.append(min(T, cuts[-1] + step))
    S = len(cuts) - 1
    seg_adapter = g.integers(0, n_adapters, S).astype(np.int32)
    seg_adapter[g.random(S) < no_adapter_frac] = -1
    if r_choices is None:
        ranks = g.integers(1, r_max + 1, n_adapters).astype(np.int32)
    else:
        ranks = g.choice(np.asarray(r_choices), n_adapters).astype(np.int32)
    scales = g.uniform(0.25, 4.0, n_adapters).astype(np.float32)
    return Workload(
        name=f"random_{seed}", seed=1000 + seed, dtype=dtype, num_layers=1,
        projs=(Proj("p", h_in, h_out, "x"),), calls=((0,),), num_tokens=T,
        seg_starts=np.asarray(cuts, np.int32), seg_adapter=seg_adapter,
        pool_size=n_adapters, ranks=ranks, scales=scales, has_base=has_base,
        r_max=r_max, description="random small case")


def mixed_case(seed: int, *, long_tokens: int = 1100, n_long: int = 2, n_short: int = 40,
               short_max: int = 3, h_in: int = 256, h_out: int = 192,
               r_choices=(8, 16, 32, 64), dtype: str = "bf16", has_base: bool = True,
               no_adapter_frac: float = 0.1, r_max: int = 64) -> Workload:
    """A continuous batch of prompts and decode steps: n_long adapters'
    prompts of long_tokens tokens in all (each at least 48 tokens, ragged,
    cut into one to three segments), interleaved in random order with n_short
    requests of 1 .. short_max tokens, each naming an adapter of its own (a
    fraction no_adapter_frac of them none)."""
    g = _rng(seed, 95)
    segs = []                                   # (adapter, tokens)
    lens = g.multinomial(long_tokens - 48 * n_long, np.full(n_long, 1.0 / n_long)) + 48
    for i, n in enumerate(lens):
        k = int(g.integers(1, 4))
        cuts = np.sort(g.choice(np.arange(1, n), k - 1, replace=False)) if k > 1 else []
        for part in np.diff(np.concatenate([[0], cuts, [n]])):
            segs.append((i, int(part)))
    for j in range(n_short):
        a = -1 if g.random() < no_adapter_frac else n_long + j
        segs.append((a, int(g.integers(1, short_max + 1))))
    segs = [segs[i] for i in g.permutation(len(segs))]
    starts = np.concatenate([[0], np.cumsum([n for _, n in segs])]).astype(np.int32)
    n_adapters = n_long + n_short
    ranks = g.choice(np.asarray(r_choices), n_adapters).astype(np.int32)
    scales = g.uniform(0.25, 4.0, n_adapters).astype(np.float32)
    return Workload(
        name=f"mixed_{seed}", seed=3000 + seed, dtype=dtype, num_layers=1,
        projs=(Proj("p", h_in, h_out, "x"),), calls=((0,),), num_tokens=int(starts[-1]),
        seg_starts=starts, seg_adapter=np.asarray([a for a, _ in segs], np.int32),
        pool_size=n_adapters, ranks=ranks, scales=scales, has_base=has_base, r_max=r_max,
        description="prompts and decode steps in one batch")


def jd_case(seed: int, *, kind: str, T: int = 96, h_in: int = 256, h_outs=(192, 64),
            n_clusters: int = 3, n_cores: int = 6, r_choices=(16, 24, 32), r_max: int = 32,
            dtype: str = "bf16", has_base: bool = True, max_seg: int = None,
            num_layers: int = 2, no_core_frac: float = 0.15) -> Workload:
    """Jointly compressed adapters: each pool entry is a cluster's shared basis
    (A_c, B_c at the cluster's rank), each segment names a cluster and one of
    n_cores cores (or -1), some segments no adapter at all.  Projections share
    one x (a q/k-like pair)."""
    g = _rng(seed, 97)
    cuts = [0]
    while cuts[-1] < T:
        step = int(g.integers(0, (max_seg or max(2, T // 6)) + 1))
        cuts.append(min(T, cuts[-1] + step))
    S = len(cuts) - 1
    seg_adapter = g.integers(0, n_clusters, S).astype(np.int32)
    seg_adapter[g.random(S) < 0.1] = -1
    seg_sigma = g.integers(0, n_cores, S).astype(np.int32)
    seg_sigma[g.random(S) < no_core_frac] = -1
    ranks = g.choice(np.asarray(r_choices), n_clusters).astype(np.int32)
    scales = g.uniform(0.5, 2.0, n_clusters).astype(np.float32)
    projs = tuple(Proj(f"p{i}", h_in, h, "x") for i, h in enumerate(h_outs))
    return Workload(
        name=f"jd_{kind}_{seed}", seed=2000 + seed, dtype=dtype, num_layers=num_layers,
        projs=projs, calls=(tuple(range(len(projs))),), num_tokens=T,
        seg_starts=np.asarray(cuts, np.int32), seg_adapter=seg_adapter,
        pool_size=n_clusters, ranks=ranks, scales=scales, has_base=has_base, r_max=r_max,
        description=f"jointly compressed adapters ({kind} cores)",
        seg_sigma=seg_sigma, n_cores=n_cores, sigma_kind=kind)


def jd_full_stack(kind: str = "full") -> Workload:
    """The full Mistral-7B stack served from jointly compressed adapters:
    1000 adapters in 10 clusters, each cluster one shared rank-32 basis per
    (layer, projection), each adapter a core; 128 decode tokens whose adapters
    follow the same bounded Zipf(1.1) draw as the plain full stack."""
    seed = 5
    base = config4()
    ids = base.seg_adapter
    clusters = (ids % 10).astype(np.int32)
    return Workload(
        name=f"jd_full_stack_{kind}", seed=seed, dtype="bf16", num_layers=LAYERS,
        projs=MISTRAL_PROJS, calls=((0, 1, 2), (3,), (4, 5), (6,)), num_tokens=128,
        seg_starts=_one_token_segments(128), seg_adapter=clusters,
        pool_size=10, ranks=np.full(10, 32, np.int32), scales=np.full(10, 1.0, np.float32),
        has_base=True, r_max=32, seg_sigma=ids.astype(np.int32), n_cores=1000,
        sigma_kind=kind,
        description=f"32 layers x 7 projections; 1000 adapters as {kind} cores over 10 shared "
                    "rank-32 bases; T=S=128, Zipf(1.1); y = base_out + delta")
