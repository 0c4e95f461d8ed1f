"""Pins for the CPU oracle, checked against what the pages and mathematics fix.

None of these re-types the oracle's loop.  Each pin compares it with
something independent: a hand-computed example, the pages' own structure
(scale 1 on the A step, the adapter scale on the B step, a float32
intermediate: "Compress then Serve", rebuttal pseudocode of
add_lora_slice_with_sigma), a merged-weight GEMM done by a library
routine, closed forms, exact-integer constructions, invariances that hold
exactly in floating point, and a textbook rounding-error bound.  The
mutation test at the end plants plausible mistakes in a copy of the oracle
and checks that the pins catch every one.
"""
import math
import os
import shutil
import subprocess
import time

import numpy as np
import pytest

import oracle
from oracle import build as oracle_build
from synth import config, random_case
from conftest import read_golden


def _delta(x, starts, segs, adapters, y_in=None, acc="f32", lib=None):
    return oracle.lora_delta(x, starts, segs, adapters, y_in, acc=acc, lib=lib)


def _rand_adapter(g, r, h_in, h_out, scale=None):
    a = g.uniform(-1, 1, (r, h_in)).astype(np.float32) / np.float32(math.sqrt(h_in))
    b = (g.standard_normal((h_out, r)) * 0.02).astype(np.float32)
    return a, b, float(np.float32(scale if scale is not None else g.uniform(0.25, 4)))


# ---------------------------------------------------------------------------
# Pins written as functions of a library handle, so the mutation test can run
# the same checks against a deliberately broken oracle.
# ---------------------------------------------------------------------------
def pin_hand_example(lib=None):
    """tests/golden/hand_tiny.txt: a worked example computed by hand."""
    rows = read_golden("hand_tiny.txt")
    kv = {}
    adapters, cur = {}, None
    x, y_in, expect = [], [], []
    for k, vals in rows:
        if k == "adapter":
            cur = int(vals[0])
            adapters[cur] = {"A": [], "B": [], "scale": float(vals[4])}
        elif k in ("A", "B"):
            adapters[cur][k].append([float(v) for v in vals])
        elif k == "x":
            x.append([float(v) for v in vals])
        elif k == "y_in":
            y_in.append([float(v) for v in vals])
        elif k == "expect":
            expect.append([float(v) for v in vals])
        else:
            kv[k] = [int(v) for v in vals]
    ad = {i: (np.array(d["A"], np.float32), np.array(d["B"], np.float32), d["scale"])
          for i, d in adapters.items()}
    for acc in ("f32", "f64"):
        y = _delta(np.array(x, np.float32), kv["seg_starts"], kv["seg_adapter"], ad,
                   np.array(y_in, np.float32), acc=acc, lib=lib)
        assert np.array_equal(y, np.array(expect)), (acc, y)


def pin_indicator_adapters(lib=None, seed=5):
    """Indicator adapters: A_i has a single 1 at [0][0], x[t][0] = 1,
    B_i[0][0] = id mod 128 and B_i[1][0] = id div 128.  Every product that
    reaches y is an exact small integer, so the output decodes, exactly, the
    adapter id each token was served with."""
    g = np.random.default_rng(seed)
    T, h_in, h_out, s = 40, 24, 16, 2.0
    ids = [3, 130, 257, 999, 77]
    adapters = {}
    for i in ids:
        r = int(g.integers(1, 9))
        a = np.zeros((r, h_in), np.float32)
        a[0, 0] = 1.0
        b = (g.standard_normal((h_out, r))).astype(np.float32)   # multiplies exact zeros
        b[:, 0] = 0.0
        b[0, 0], b[1, 0] = i % 128, i // 128
        adapters[i] = (a, b, s)
    cuts = np.sort(g.choice(np.arange(1, T), 9, replace=False))
    starts = np.concatenate([[0], cuts, [T]]).astype(np.int32)
    segs = g.choice(ids + [-1], len(starts) - 1).astype(np.int32)
    x = g.standard_normal((T, h_in)).astype(np.float32)
    x[:, 0] = 1.0
    y = _delta(x, starts, segs, adapters, lib=lib)
    expect_id = np.full(T, -1)
    for si in range(len(segs)):
        for t in range(starts[si], starts[si + 1]):
            expect_id[t] = segs[si]
    for t in range(T):
        if expect_id[t] == -1:
            assert np.all(y[t] == 0), t
        else:
            got = int(y[t, 0] / s) + 128 * int(y[t, 1] / s)
            assert got == expect_id[t] and y[t, 0] == s * (expect_id[t] % 128), (t, got)
            assert np.all(y[t, 2:] == 0), t


def pin_merged_weight(lib=None, seed=7):
    """One adapter for every token: y = W x + s B (A x) must equal the
    merged-weight product (W + s B A) x, evaluated by numpy in float64.
    W and x are small integers so y_in = W x is exact in float32."""
    g = np.random.default_rng(seed)
    T, h_in, h_out, r, s = 12, 40, 24, 5, 1.5
    W = g.integers(-3, 4, (h_out, h_in)).astype(np.float64)
    x = g.integers(-4, 5, (T, h_in)).astype(np.float32)
    a, b, _ = _rand_adapter(g, r, h_in, h_out)
    y_in = (x.astype(np.float64) @ W.T).astype(np.float32)
    starts = np.array([0, 5, 5, T], np.int32)             # includes an empty segment
    segs = np.array([4, 4, 4], np.int32)
    merged = (W + s * b.astype(np.float64) @ a.astype(np.float64))
    ref = x.astype(np.float64) @ merged.T
    y64 = _delta(x, starts, segs, {4: (a, b, s)}, y_in, acc="f64", lib=lib)
    y32 = _delta(x, starts, segs, {4: (a, b, s)}, y_in, acc="f32", lib=lib)
    scale = np.abs(ref).max()
    assert np.abs(y64 - ref).max() <= 1e-12 * scale
    assert np.abs(y32 - ref).max() <= 1e-5 * scale


def pin_b_zero(lib=None, seed=11):
    """B = 0 gives a zero delta: y equals y_in, value for value."""
    w = random_case(seed, T=48, h_in=64, h_out=40)
    g = np.random.default_rng(seed)
    x = g.standard_normal((w.num_tokens, 64)).astype(np.float32)
    y_in = g.standard_normal((w.num_tokens, 40)).astype(np.float32)
    adapters = {}
    for i in range(w.pool_size):
        a, _, s = _rand_adapter(g, int(w.ranks[i]), 64, 40)
        adapters[i] = (a, np.zeros((40, int(w.ranks[i])), np.float32), s)
    for acc in ("f32", "f64"):
        y = _delta(x, w.seg_starts, w.seg_adapter, adapters, y_in, acc=acc, lib=lib)
        assert np.array_equal(y, y_in)


def _sigma_case(seed, *, r=6, h_in=40, h_out=24, T=30, n_clusters=3, n_cores=5):
    """A small batch of jointly compressed adapters: shared bases per cluster
    (ids 10, 11, ...), cores 0..n_cores-1, segment (cluster, core) pairs,
    some segments without an adapter or without a core."""
    g = np.random.default_rng(seed)
    bases = {10 + c: _rand_adapter(g, r, h_in, h_out) for c in range(n_clusters)}
    cuts = np.sort(g.choice(np.arange(1, T), 7, replace=False))
    starts = np.concatenate([[0], cuts, [T]]).astype(np.int32)
    S = len(starts) - 1
    segs = g.choice(list(bases) + [-1], S).astype(np.int32)
    sig = g.integers(-1, n_cores, S).astype(np.int32)
    x = g.standard_normal((T, h_in)).astype(np.float32)
    return g, x, starts, segs, sig, bases


def pin_sigma_identity(lib=None, seed=21):
    """No core, and the identity core (full and diagonal), both reduce the
    three steps to plain LoRA: the same values, bit for bit, as the two-step
    delta with the shared basis as the adapter."""
    g, x, starts, segs, sig, bases = _sigma_case(seed)
    r = 6
    y_in = g.standard_normal((x.shape[0], 24)).astype(np.float32)
    for acc in ("f32", "f64"):
        plain = _delta(x, starts, segs, bases, y_in, acc=acc, lib=lib)
        none = oracle.lora_delta_sigma(x, starts, segs, np.full_like(sig, -1), bases,
                                       np.zeros((1, r, r), np.float32), "full", y_in,
                                       acc=acc, lib=lib)
        eye = oracle.lora_delta_sigma(x, starts, segs, np.maximum(sig, 0), bases,
                                      np.stack([np.eye(r, dtype=np.float32)] * 5), "full",
                                      y_in, acc=acc, lib=lib)
        ones = oracle.lora_delta_sigma(x, starts, segs, np.maximum(sig, 0), bases,
                                       np.ones((5, r), np.float32), "diag", y_in, acc=acc,
                                       lib=lib)
        for got in (none, eye, ones):
            assert np.array_equal(got, plain), acc


def pin_sigma_diag_powers_of_two(lib=None, seed=23):
    """A diagonal core of powers of two scales rank row j of v exactly, so
    the three steps equal plain LoRA with A's row j scaled by the same power
    of two, bit for bit (each segment's core applied to its own copy of A)."""
    g, x, starts, segs, sig, bases = _sigma_case(seed)
    r = 6
    cores = (2.0 ** g.integers(-3, 4, (5, r))).astype(np.float32)
    for acc in ("f32", "f64"):
        got = oracle.lora_delta_sigma(x, starts, segs, sig, bases, cores, "diag",
                                      acc=acc, lib=lib)
        for si in range(len(segs)):
            a0, b0 = starts[si], starts[si + 1]
            if segs[si] < 0 or a0 == b0:
                continue
            a, b, s = bases[int(segs[si])]
            if sig[si] >= 0:
                a = (a * cores[sig[si]][:, None]).astype(np.float32)
            ref = _delta(x[a0:b0], [0, b0 - a0], [7], {7: (a, b, s)}, acc=acc, lib=lib)
            assert np.array_equal(got[a0:b0], ref), (acc, si)


def pin_sigma_full_merged(lib=None, seed=29):
    """A full core: the delta equals the merged product s (B Sigma A) x done
    by numpy in float64, and a full core that is diagonal equals the
    diagonal kind exactly."""
    g, x, starts, segs, sig, bases = _sigma_case(seed)
    r = 6
    cores = g.standard_normal((5, r, r)).astype(np.float32)
    y64 = oracle.lora_delta_sigma(x, starts, segs, sig, bases, cores, "full", acc="f64",
                                  lib=lib)
    y32 = oracle.lora_delta_sigma(x, starts, segs, sig, bases, cores, "full", acc="f32",
                                  lib=lib)
    ref = np.zeros_like(y64)
    for si in range(len(segs)):
        a0, b0 = starts[si], starts[si + 1]
        if segs[si] < 0:
            continue
        a, b, s = (m.astype(np.float64) if isinstance(m, np.ndarray) else m
                   for m in bases[int(segs[si])])
        core = np.eye(r) if sig[si] < 0 else cores[sig[si]].astype(np.float64)
        ref[a0:b0] = x[a0:b0].astype(np.float64) @ (s * b @ core @ a).T
    scale = np.abs(ref).max()
    assert np.abs(y64 - ref).max() <= 1e-12 * scale
    assert np.abs(y32 - ref).max() <= 1e-5 * scale
    d = g.standard_normal((5, r)).astype(np.float32)
    full = np.stack([np.diag(v) for v in d]).astype(np.float32)
    for acc in ("f32", "f64"):
        assert np.array_equal(
            oracle.lora_delta_sigma(x, starts, segs, sig, bases, full, "full", acc=acc, lib=lib),
            oracle.lora_delta_sigma(x, starts, segs, sig, bases, d, "diag", acc=acc, lib=lib))


def _merge_case(seed, *, K=3, T=36, h_in=40, h_out=24, n_adapters=5):
    g = np.random.default_rng(seed)
    adapters = {i: _rand_adapter(g, int(g.integers(1, 9)), h_in, h_out) for i in range(n_adapters)}
    cuts = np.sort(g.choice(np.arange(1, T), 6, replace=False))
    starts = np.concatenate([[0], cuts, [T]]).astype(np.int32)
    S = len(starts) - 1
    seg_ad = g.integers(-1, n_adapters, (S, K)).astype(np.int32)
    seg_w = g.uniform(-1.5, 1.5, (S, K)).astype(np.float32)
    x = g.standard_normal((T, h_in)).astype(np.float32)
    y_in = g.standard_normal((T, h_out)).astype(np.float32)
    return g, x, starts, seg_ad, seg_w, adapters, y_in


def pin_merge_one_slot(lib=None, seed=41):
    """One slot of weight 1 is the plain delta, bit for bit; a slot of weight
    2^e equals the plain delta of that adapter with its scale times 2^e."""
    g, x, starts, seg_ad, seg_w, adapters, y_in = _merge_case(seed, K=1)
    for acc in ("f32", "f64"):
        ones = np.ones_like(seg_w)
        assert np.array_equal(
            oracle.lora_delta_merge(x, starts, seg_ad, ones, adapters, y_in, acc=acc, lib=lib),
            _delta(x, starts, seg_ad[:, 0], adapters, y_in, acc=acc, lib=lib))
        e = int(g.integers(-3, 4))
        pw = np.full_like(seg_w, 2.0 ** e)
        scaled = {i: (a, b, s * 2.0 ** e) for i, (a, b, s) in adapters.items()}
        assert np.array_equal(
            oracle.lora_delta_merge(x, starts, seg_ad, pw, adapters, y_in, acc=acc, lib=lib),
            _delta(x, starts, seg_ad[:, 0], scaled, y_in, acc=acc, lib=lib))


def pin_merge_slots_in_order(lib=None, seed=43):
    """K slots equal K plain deltas applied one after the other (each on the
    previous result), with the scales times power-of-two weights: bit for bit."""
    g, x, starts, seg_ad, seg_w, adapters, y_in = _merge_case(seed, K=3)
    pw = (2.0 ** g.integers(-2, 3, seg_w.shape)).astype(np.float32)
    for acc in ("f32",):
        got = oracle.lora_delta_merge(x, starts, seg_ad, pw, adapters, y_in, acc=acc, lib=lib)
        y = y_in
        for k in range(seg_ad.shape[1]):
            # per segment, the slot's adapter at its weighted scale: one
            # adapter id per (segment, slot) pair
            ad, segs = {}, []
            for si in range(len(seg_ad)):
                a = int(seg_ad[si, k])
                if a < 0:
                    segs.append(-1)
                    continue
                key = 1000 * si + a
                A, B, s = adapters[a]
                ad[key] = (A, B, float(np.float32(pw[si, k]) * np.float32(s)))
                segs.append(key)
            y = _delta(x, starts, segs, ad, y, acc=acc, lib=lib) if ad else y
        assert np.array_equal(got, y)


def pin_merge_merged_weight(lib=None, seed=47):
    """The merge equals x (sum_k w_k s_k B_k A_k)^T per segment, by numpy in
    float64; a weight of 0 leaves y_in."""
    g, x, starts, seg_ad, seg_w, adapters, y_in = _merge_case(seed, K=3)
    y64 = oracle.lora_delta_merge(x, starts, seg_ad, seg_w, adapters, y_in, acc="f64", lib=lib)
    ref = y_in.astype(np.float64).copy()
    for si in range(len(seg_ad)):
        W = np.zeros((24, 40))
        for k in range(seg_ad.shape[1]):
            a = int(seg_ad[si, k])
            if a >= 0:
                A, B, s = adapters[a]
                W += float(seg_w[si, k]) * s * (B.astype(np.float64) @ A.astype(np.float64))
        ref[starts[si]:starts[si + 1]] += x[starts[si]:starts[si + 1]].astype(np.float64) @ W.T
    assert np.abs(y64 - ref).max() <= 1e-12 * np.abs(ref).max()
    zero = oracle.lora_delta_merge(x, starts, seg_ad, np.zeros_like(seg_w), adapters, y_in,
                                   acc="f32", lib=lib)
    assert np.all(zero == y_in)


ALL_PINS = (pin_hand_example, pin_indicator_adapters, pin_merged_weight, pin_b_zero,
            pin_sigma_identity, pin_sigma_diag_powers_of_two, pin_sigma_full_merged,
            pin_merge_one_slot, pin_merge_slots_in_order, pin_merge_merged_weight)


def test_hand_example():
    pin_hand_example()


def test_indicator_adapters():
    pin_indicator_adapters()


def test_merged_weight():
    pin_merged_weight()


def test_b_zero_identity():
    pin_b_zero()


def test_rank1_closed_form():
    """Rank 1: delta[t] = s * b * (a . x[t]); the dot product is taken with
    math.fsum (correctly rounded), so the float64 oracle must agree to a few
    ulps."""
    g = np.random.default_rng(3)
    T, h_in, h_out = 9, 200, 33
    a, b, s = _rand_adapter(g, 1, h_in, h_out)
    x = g.standard_normal((T, h_in)).astype(np.float32)
    y = _delta(x, [0, T], [0], {0: (a, b, s)}, acc="f64")
    for t in range(T):
        dot = math.fsum(float(a[0, k]) * float(x[t, k]) for k in range(h_in))
        ref = np.array([s * float(b[o, 0]) * dot for o in range(h_out)])
        assert np.allclose(y[t], ref, rtol=1e-13, atol=1e-15)


def test_brute_force_matmul():
    """Per segment, delta = s * (X_seg A^T) B^T, via numpy float64 matmul, on
    the tiny fp32 workload and on random heterogeneous batches."""
    cases = [config(0)] + [random_case(i) for i in range(6)]
    for w in cases:
        pr = w.projs[0]
        x = w.activation(0, pr.x_key)
        y64 = oracle.workload_call(w, 0, 0, acc="f64")
        ref = np.zeros((w.num_tokens, pr.h_out))
        for si in range(w.num_segs):
            aid = int(w.seg_adapter[si])
            lo, hi = int(w.seg_starts[si]), int(w.seg_starts[si + 1])
            if aid < 0 or hi == lo:
                continue
            a, b = w.adapter_block(aid, 0, 0)
            ref[lo:hi] = float(w.scales[aid]) * (
                (x[lo:hi].astype(np.float64) @ a.T.astype(np.float64)) @ b.T.astype(np.float64))
        assert np.allclose(y64, ref, rtol=1e-12, atol=1e-14), w.name


def test_permutation_invariance():
    """Reordering segments (with their token rows) changes no token's result,
    bit for bit."""
    for seed in range(4):
        w = random_case(seed, T=60, h_in=96, h_out=48)
        x = w.activation(0, "x")
        y = oracle.workload_call(w, 0, 0)
        perm = np.random.default_rng(seed).permutation(w.num_segs)
        rows, new_starts = [], [0]
        for si in perm:
            rows.extend(range(w.seg_starts[si], w.seg_starts[si + 1]))
            new_starts.append(new_starts[-1] + w.seg_starts[si + 1] - w.seg_starts[si])
        ad = {i: (*w.adapter_block(i, 0, 0), float(w.scales[i])) for i in range(w.pool_size)}
        y2 = _delta(x[rows], new_starts, w.seg_adapter[perm], ad)
        assert np.array_equal(y2, y[rows])


def test_segment_split_invariance():
    """Cutting a segment in two with the same adapter is bit-identical."""
    w = random_case(21, T=50, h_in=64, h_out=32, max_seg=20)
    x = w.activation(0, "x")
    ad = {i: (*w.adapter_block(i, 0, 0), float(w.scales[i])) for i in range(w.pool_size)}
    y = _delta(x, w.seg_starts, w.seg_adapter, ad)
    starts, segs = [0], []
    for si in range(w.num_segs):
        lo, hi = int(w.seg_starts[si]), int(w.seg_starts[si + 1])
        mid = (lo + hi) // 2
        starts += [mid, hi]
        segs += [w.seg_adapter[si]] * 2
    y2 = _delta(x, starts, segs, ad)
    assert np.array_equal(y, y2)


def test_padding_invariance():
    """An adapter of rank r stored with zero rows of A and zero columns of B
    up to a larger rank gives the same bits (the extra products are +-0)."""
    g = np.random.default_rng(8)
    T, h_in, h_out = 20, 48, 40
    x = g.standard_normal((T, h_in)).astype(np.float32)
    y_in = g.standard_normal((T, h_out)).astype(np.float32)
    for r, r_pad in ((1, 8), (5, 8), (12, 16), (33, 64)):
        a, b, s = _rand_adapter(g, r, h_in, h_out)
        ap = np.zeros((r_pad, h_in), np.float32)
        ap[:r] = a
        bp = np.zeros((h_out, r_pad), np.float32)
        bp[:, :r] = b
        y = _delta(x, [0, T], [1], {1: (a, b, s)}, y_in)
        yp = _delta(x, [0, T], [1], {1: (ap, bp, s)}, y_in)
        assert np.array_equal(y, yp), (r, r_pad)


def test_linearity():
    """delta(2x) = 2 delta(x) and delta with 2s = 2 delta with s (exact: powers
    of two); splitting the rank, (A, B) = ([A1; A2], [B1 B2]), adds the two
    halves' deltas (to rounding)."""
    g = np.random.default_rng(9)
    T, h_in, h_out, r = 16, 80, 24, 12
    x = g.standard_normal((T, h_in)).astype(np.float32)
    a, b, s = _rand_adapter(g, r, h_in, h_out, scale=1.25)
    y = _delta(x, [0, T], [0], {0: (a, b, s)})
    assert np.array_equal(_delta(2 * x, [0, T], [0], {0: (a, b, s)}), 2 * y)
    assert np.array_equal(_delta(x, [0, T], [0], {0: (a, b, 2 * s)}), 2 * y)
    y64 = _delta(x, [0, T], [0], {0: (a, b, s)}, acc="f64")
    h1 = _delta(x, [0, T], [0], {0: (a[:5], b[:, :5], s)}, acc="f64")
    h2 = _delta(x, [0, T], [0], {0: (a[5:], b[:, 5:], s)}, acc="f64")
    assert np.allclose(h1 + h2, y64, rtol=1e-12, atol=1e-15)


def test_f32_within_rounding_bound():
    """The float32 oracle stays inside the textbook bound for recursive
    summation (|fl(sum) - sum| <= gamma_n * sum|terms|, gamma_n = n u / (1 - n u),
    u = 2^-24), propagated through the A step, the B step, the scale and the
    add, measured against the float64 oracle."""
    u = 2.0 ** -24
    gam = lambda n: n * u / (1 - n * u)  # noqa: E731
    for w in [config(0)] + [random_case(i, has_base=True) for i in (1, 2, 3)]:
        pr = w.projs[0]
        x = w.activation(0, pr.x_key).astype(np.float64)
        g = np.random.default_rng(w.seed)
        y_in = g.standard_normal((w.num_tokens, pr.h_out)).astype(np.float32)
        ad = {i: (*w.adapter_block(i, 0, 0), float(w.scales[i])) for i in range(w.pool_size)}
        y32 = _delta(w.activation(0, pr.x_key), w.seg_starts, w.seg_adapter, ad, y_in)
        y64 = _delta(w.activation(0, pr.x_key), w.seg_starts, w.seg_adapter, ad, y_in, acc="f64")
        tok = w.token_adapter()
        for t in range(w.num_tokens):
            i = int(tok[t])
            if i < 0:
                assert np.array_equal(y32[t], y_in[t])
                continue
            a, b, s = ad[i]
            a, b = a.astype(np.float64), b.astype(np.float64)
            r = a.shape[0]
            v = a @ x[t]
            ev = gam(pr.h_in) * (np.abs(a) @ np.abs(x[t]))            # A-step error
            d = b @ v
            ed = gam(r) * (np.abs(b) @ (np.abs(v) + ev)) + np.abs(b) @ ev
            sd = abs(s) * (np.abs(d) + ed)
            bound = abs(s) * ed + u * sd + u * (np.abs(y_in[t]) + sd) * 1.0001 + 1e-30
            assert np.all(np.abs(y32[t] - y64[t]) <= bound), (w.name, t)


def test_sigma_identity():
    pin_sigma_identity()


def test_sigma_diag_powers_of_two():
    pin_sigma_diag_powers_of_two()


def test_sigma_full_merged():
    pin_sigma_full_merged()


def test_merge_one_slot():
    pin_merge_one_slot()


def test_merge_slots_in_order():
    pin_merge_slots_in_order()


def test_merge_merged_weight():
    pin_merge_merged_weight()


def test_sigma_errors():
    g, x, starts, segs, sig, bases = _sigma_case(31)
    bad = sig.copy()
    bad[0] = 5                                            # core index out of range
    with pytest.raises(oracle.OracleError):
        oracle.lora_delta_sigma(x, starts, segs, bad, bases, np.ones((5, 6), np.float32), "diag")


def test_errors():
    x = np.zeros((4, 8), np.float32)
    ad = {1: (np.zeros((2, 8), np.float32), np.zeros((8, 2), np.float32), 1.0)}
    for starts, segs in (([0, 3], [1]), ([1, 4], [1]), ([0, 3, 2, 4], [1, 1, 1]), ([0, 4], [2])):
        with pytest.raises(oracle.OracleError):
            _delta(x, starts, segs, ad)


def test_config0_under_one_second():
    """The tiny fp32 workload's oracle run finishes in under a second."""
    w = config(0)
    t0 = time.perf_counter()
    oracle.workload_call(w, 0, 0)
    assert time.perf_counter() - t0 < 1.0


# ---------------------------------------------------------------------------
# Mutation test: each planted mistake must make at least one pin fail.
# ---------------------------------------------------------------------------
MUTATIONS = {
    "drop_scale": ("yt[o] = yt[o] + sc * d;", "yt[o] = yt[o] + d;"),
    "transpose_B": ("const float *bo = B[a] + (int64_t)o * r;\n"
                    "            float d = 0.0f;", None),
    "rank_off_by_one": ("for (int32_t j = 0; j < r; ++j) {\n            float acc",
                        "for (int32_t j = 0; j < r - 1; ++j) {\n            float acc"),
    "reversed_x": ("acc += aj[k] * xt[k];", "acc += aj[k] * xt[h_in - 1 - k];"),
    "drop_y_in": ("yt[o] = y_in ? y_in[(int64_t)t * ld_in + o] : 0.0f;", "yt[o] = 0.0f;"),
    "wrong_lookup": ("if (ids[a] == id) return a;", "if (ids[a] == id) return (a + 1) % n;"),
    "sign_flip": ("yt[o] = yt[o] + sc * d;", "yt[o] = yt[o] - sc * d;"),
    "no_adapter_uses_first": ("const int32_t a = tok_a[t];",
                              "const int32_t a = tok_a[t] < 0 ? 0 : tok_a[t];"),
    "sigma_transposed": ("acc += row[k] * v[k];",
                         "acc += sigma[sj][(int64_t)k * sigma_ld + j] * v[k];"),
    "sigma_skipped": ("u[j] = acc;", "u[j] = v[j];"),
    "sigma_diag_ignored": ("u[j] = sigma[sj][j] * v[j];", "u[j] = v[j];"),
    "sigma_first_core": ("const int32_t sj = tok_s[t];",
                         "const int32_t sj = tok_s[t] < 0 ? -1 : 0;"),
    "sigma_b_reads_buffer": ("for (int32_t j = 0; j < r; ++j) d += bo[j] * u[j];",
                             "for (int32_t j = 0; j < r; ++j) d += bo[j] * v[j];"),
    "merge_weight_dropped": ("const float sw = seg_weights[s * K + k] * scales[a];",
                             "const float sw = scales[a];"),
    "merge_first_slot_only": ("for (int32_t k = 0; k < K; ++k) {\n                const int32_t a = slot_a",
                              "for (int32_t k = 0; k < 1; ++k) {\n                const int32_t a = slot_a"),
    "merge_y_in_per_slot": ("yt[o] = yt[o] + sw * d;",
                            "yt[o] = (y_in ? y_in[(int64_t)t * ld_in + o] : 0.0f) + sw * d;"),
}


def _mutate(src, name):
    old, new = MUTATIONS[name]
    if name == "transpose_B":
        # read B as if it were stored r x h_out
        old = "d += bo[j] * v[j];"
        new = "d += B[a][(int64_t)j * h_out + o] * v[j];"
    assert src.count(old) >= 1, name
    return src.replace(old, new, 1)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(oracle_build.SRC).read()
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(_mutate(src, name))
    lib_path = str(tmp_path / "liboracle_mut.so")
    oracle_build.build(out=lib_path, src=str(mutated))
    lib = oracle.load_library(lib_path)
    failures = 0
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, oracle.OracleError):
            failures += 1
    assert failures >= 1, f"no pin caught mutation {name}"
