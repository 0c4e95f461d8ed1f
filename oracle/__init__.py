"""CPU oracle for the multi-adapter LoRA delta -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path never does; the oracle shares no
code with the GPU library.

``lora_delta`` runs the plain per-token loop of ``oracle.c``:

    y[t] = y_in[t] + s_i * B_i (A_i x[t])

for one adapted linear layer of a heterogeneous batch ("TGI Multi-LoRA:
Deploy Once, Serve 30 Models", "Technical Foundation" and "How Multi-LoRA
Serving Works"; "Compress then Serve", rebuttal pseudocode of
add_lora_slice_with_sigma, steps 1 and 3).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


def load_library(path):
    """Load a compiled oracle library and declare its signatures."""
    lib = ctypes.CDLL(path)
    _vpp = ctypes.POINTER(ctypes.c_void_p)
    for name, yp in (("oracle_delta_f32", _f32p), ("oracle_delta_f64", _f64p)):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                       _f32p, ctypes.c_int64,
                       ctypes.c_int32, _i32p, _i32p,
                       ctypes.c_int32, _i32p, _i32p, _f32p,
                       _vpp, _vpp,
                       _f32p, ctypes.c_int64,
                       yp, ctypes.c_int64, ctypes.c_int32]
    for name, yp in (("oracle_delta_sigma_f32", _f32p), ("oracle_delta_sigma_f64", _f64p)):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                       _f32p, ctypes.c_int64,
                       ctypes.c_int32, _i32p, _i32p, _i32p,
                       ctypes.c_int32, _i32p, _i32p, _f32p,
                       _vpp, _vpp,
                       ctypes.c_int32, ctypes.c_int32, _vpp, ctypes.c_int64,
                       _f32p, ctypes.c_int64,
                       yp, ctypes.c_int64, ctypes.c_int32]
    for name, yp in (("oracle_delta_merge_f32", _f32p), ("oracle_delta_merge_f64", _f64p)):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                       _f32p, ctypes.c_int64,
                       ctypes.c_int32, _i32p, ctypes.c_int32, _i32p, _f32p,
                       ctypes.c_int32, _i32p, _i32p, _f32p,
                       _vpp, _vpp,
                       _f32p, ctypes.c_int64,
                       yp, ctypes.c_int64, ctypes.c_int32]
    return lib


def _load():
    """The built oracle, or the build HAB_ORACLE_LIB names (e.g. a sanitizer
    build for the tests)."""
    global _lib
    if _lib is None:
        path = os.environ.get("HAB_ORACLE_LIB")
        if not path:
            path = _build.LIB
            if not os.path.exists(path):
                _build.build()
        _lib = load_library(path)
    return _lib


class OracleError(RuntimeError):
    pass


def lora_delta(x, seg_starts, seg_adapter, adapters, y_in=None, *, acc="f32", threads=1,
               lib=None):
    """One adapted linear layer over a heterogeneous batch.

    x:           [T][h_in] float32 (bf16 inputs passed as their exact float32 values)
    seg_starts:  [S+1] int32, seg_adapter: [S] int32 (-1 = no adapter)
    adapters:    {id: (A [r][h_in], B [h_out][r], scale)}
    y_in:        [T][h_out] float32 or None (zero)
    acc:         "f32" (float accumulation) or "f64" (double accumulation)
    lib:         a library from ``load_library`` (default: the built oracle)
    Returns y [T][h_out] as float32 or float64.
    """
    lib = lib or _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    T, h_in = x.shape
    seg_starts = np.ascontiguousarray(seg_starts, dtype=np.int32)
    seg_adapter = np.ascontiguousarray(seg_adapter, dtype=np.int32)
    ids = np.asarray(sorted(adapters), dtype=np.int32)
    mats = [(np.ascontiguousarray(adapters[i][0], dtype=np.float32),
             np.ascontiguousarray(adapters[i][1], dtype=np.float32)) for i in ids]
    if mats:
        h_out = mats[0][1].shape[0]
    elif y_in is not None:
        h_out = np.asarray(y_in).shape[1]
    else:
        raise ValueError("h_out unknown: no adapters and no y_in")
    for a, b in mats:
        if a.shape[1] != h_in or b.shape[0] != h_out or a.shape[0] != b.shape[1]:
            raise ValueError("adapter shapes do not match x / each other")
    ranks = np.asarray([a.shape[0] for a, _ in mats], dtype=np.int32)
    scales = np.asarray([adapters[i][2] for i in ids], dtype=np.float32)
    n = len(ids)
    a_ptrs = (ctypes.c_void_p * max(n, 1))(*[m[0].ctypes.data for m in mats])
    b_ptrs = (ctypes.c_void_p * max(n, 1))(*[m[1].ctypes.data for m in mats])
    if y_in is not None:
        y_in = np.ascontiguousarray(y_in, dtype=np.float32)
        if y_in.shape != (T, h_out):
            raise ValueError("y_in shape")
        yin_p, ld_in = y_in.ctypes.data_as(_f32p), h_out
    else:
        yin_p, ld_in = None, 0
    if acc == "f32":
        y = np.empty((T, h_out), dtype=np.float32)
        fn, yp = lib.oracle_delta_f32, y.ctypes.data_as(_f32p)
    elif acc == "f64":
        y = np.empty((T, h_out), dtype=np.float64)
        fn, yp = lib.oracle_delta_f64, y.ctypes.data_as(_f64p)
    else:
        raise ValueError(acc)
    rc = fn(T, h_in, h_out, x.ctypes.data_as(_f32p), h_in,
            int(seg_adapter.shape[0]), seg_starts.ctypes.data_as(_i32p),
            seg_adapter.ctypes.data_as(_i32p),
            n, ids.ctypes.data_as(_i32p), ranks.ctypes.data_as(_i32p),
            scales.ctypes.data_as(_f32p), a_ptrs, b_ptrs,
            yin_p, ld_in, yp, h_out, int(threads))
    if rc != 0:
        raise OracleError("malformed segment table or unknown adapter id")
    return y


def lora_delta_sigma(x, seg_starts, seg_adapter, seg_sigma, adapters, cores, kind,
                     y_in=None, *, acc="f32", threads=1, lib=None):
    """The three-step delta of jointly compressed adapters ("Compress then
    Serve", rebuttal pseudocode of add_lora_slice_with_sigma, steps 1-3):
    y[t] = y_in[t] + s_c * B_c (Sigma_j (A_c x[t])).

    adapters:   {id: (A_c [r][h_in], B_c [h_out][r], scale)}: the shared bases
    seg_sigma:  [S] int32 core index per segment (-1: no core)
    cores:      [n][r][r] ("full", JD-Full) or [n][r] ("diag", JD-Diag), float32
    Other arguments as ``lora_delta``.
    """
    lib = lib or _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    T, h_in = x.shape
    seg_starts = np.ascontiguousarray(seg_starts, dtype=np.int32)
    seg_adapter = np.ascontiguousarray(seg_adapter, dtype=np.int32)
    seg_sigma = np.ascontiguousarray(seg_sigma, dtype=np.int32)
    if seg_sigma.shape != seg_adapter.shape:
        raise ValueError("seg_sigma shape")
    kind_code = {"diag": 1, "full": 2}[kind]
    cores = np.ascontiguousarray(cores, dtype=np.float32)
    n_sig = cores.shape[0]
    ids = np.asarray(sorted(adapters), dtype=np.int32)
    mats = [(np.ascontiguousarray(adapters[i][0], dtype=np.float32),
             np.ascontiguousarray(adapters[i][1], dtype=np.float32)) for i in ids]
    if mats:
        h_out = mats[0][1].shape[0]
    elif y_in is not None:
        h_out = np.asarray(y_in).shape[1]
    else:
        raise ValueError("h_out unknown: no adapters and no y_in")
    for a, b in mats:
        if a.shape[1] != h_in or b.shape[0] != h_out or a.shape[0] != b.shape[1]:
            raise ValueError("adapter shapes do not match x / each other")
        if a.shape[0] > cores.shape[1] or (kind == "full" and a.shape[0] > cores.shape[2]):
            raise ValueError("cores smaller than an adapter's rank")
    ranks = np.asarray([a.shape[0] for a, _ in mats], dtype=np.int32)
    scales = np.asarray([adapters[i][2] for i in ids], dtype=np.float32)
    n = len(ids)
    a_ptrs = (ctypes.c_void_p * max(n, 1))(*[m[0].ctypes.data for m in mats])
    b_ptrs = (ctypes.c_void_p * max(n, 1))(*[m[1].ctypes.data for m in mats])
    s_ptrs = (ctypes.c_void_p * max(n_sig, 1))(*[cores[j].ctypes.data for j in range(n_sig)])
    sigma_ld = cores.shape[2] if kind == "full" else 0
    if y_in is not None:
        y_in = np.ascontiguousarray(y_in, dtype=np.float32)
        if y_in.shape != (T, h_out):
            raise ValueError("y_in shape")
        yin_p, ld_in = y_in.ctypes.data_as(_f32p), h_out
    else:
        yin_p, ld_in = None, 0
    if acc == "f32":
        y = np.empty((T, h_out), dtype=np.float32)
        fn, yp = lib.oracle_delta_sigma_f32, y.ctypes.data_as(_f32p)
    elif acc == "f64":
        y = np.empty((T, h_out), dtype=np.float64)
        fn, yp = lib.oracle_delta_sigma_f64, y.ctypes.data_as(_f64p)
    else:
        raise ValueError(acc)
    rc = fn(T, h_in, h_out, x.ctypes.data_as(_f32p), h_in,
            int(seg_adapter.shape[0]), seg_starts.ctypes.data_as(_i32p),
            seg_adapter.ctypes.data_as(_i32p), seg_sigma.ctypes.data_as(_i32p),
            n, ids.ctypes.data_as(_i32p), ranks.ctypes.data_as(_i32p),
            scales.ctypes.data_as(_f32p), a_ptrs, b_ptrs,
            n_sig, kind_code, s_ptrs, sigma_ld,
            yin_p, ld_in, yp, h_out, int(threads))
    if rc != 0:
        raise OracleError("malformed segment table, unknown adapter id or core index")
    return y


def lora_delta_merge(x, seg_starts, seg_adapters, seg_weights, adapters, y_in=None, *,
                     acc="f32", threads=1, lib=None):
    """Weighted merge of several adapters per request ("predibase/lorax":
    adapters merged per request into a weighted ensemble):
    y[t] = y_in[t] + sum_k (w_k s_k) B_k (A_k x[t]), slot by slot.

    seg_adapters, seg_weights: [S][K] int32 / float32 (adapter -1: empty slot)
    Other arguments as ``lora_delta``.
    """
    lib = lib or _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    T, h_in = x.shape
    seg_starts = np.ascontiguousarray(seg_starts, dtype=np.int32)
    seg_adapters = np.ascontiguousarray(seg_adapters, dtype=np.int32)
    seg_weights = np.ascontiguousarray(seg_weights, dtype=np.float32)
    if seg_adapters.ndim != 2 or seg_weights.shape != seg_adapters.shape:
        raise ValueError("seg_adapters and seg_weights must both be [S][K]")
    S, K = seg_adapters.shape
    ids = np.asarray(sorted(adapters), dtype=np.int32)
    mats = [(np.ascontiguousarray(adapters[i][0], dtype=np.float32),
             np.ascontiguousarray(adapters[i][1], dtype=np.float32)) for i in ids]
    if mats:
        h_out = mats[0][1].shape[0]
    elif y_in is not None:
        h_out = np.asarray(y_in).shape[1]
    else:
        raise ValueError("h_out unknown: no adapters and no y_in")
    ranks = np.asarray([a.shape[0] for a, _ in mats], dtype=np.int32)
    scales = np.asarray([adapters[i][2] for i in ids], dtype=np.float32)
    n = len(ids)
    a_ptrs = (ctypes.c_void_p * max(n, 1))(*[m[0].ctypes.data for m in mats])
    b_ptrs = (ctypes.c_void_p * max(n, 1))(*[m[1].ctypes.data for m in mats])
    if y_in is not None:
        y_in = np.ascontiguousarray(y_in, dtype=np.float32)
        yin_p, ld_in = y_in.ctypes.data_as(_f32p), h_out
    else:
        yin_p, ld_in = None, 0
    if acc == "f32":
        y = np.empty((T, h_out), dtype=np.float32)
        fn, yp = lib.oracle_delta_merge_f32, y.ctypes.data_as(_f32p)
    else:
        y = np.empty((T, h_out), dtype=np.float64)
        fn, yp = lib.oracle_delta_merge_f64, y.ctypes.data_as(_f64p)
    rc = fn(T, h_in, h_out, x.ctypes.data_as(_f32p), h_in, int(S),
            seg_starts.ctypes.data_as(_i32p), int(K), seg_adapters.ctypes.data_as(_i32p),
            seg_weights.ctypes.data_as(_f32p), n, ids.ctypes.data_as(_i32p),
            ranks.ctypes.data_as(_i32p), scales.ctypes.data_as(_f32p), a_ptrs, b_ptrs,
            yin_p, ld_in, yp, h_out, int(threads))
    if rc != 0:
        raise OracleError("malformed segment table or unknown adapter id")
    return y


def workload_call(w, layer, p, *, acc="f32", threads=1, tokens=None):
    """Oracle result for projection ``p`` of ``layer`` of a synth Workload.

    y_in is base_out when the workload gives one, else zero.  ``tokens``
    restricts the evaluation to a subset of token rows (each row only depends
    on its own x row, adapter and y_in row), returning rows in that order.
    """
    pr = w.projs[p]
    x = w.activation(layer, pr.x_key)
    y_in = w.base_out(layer, p) if w.has_base else None
    starts, segs = w.seg_starts, w.seg_adapter
    if tokens is not None:
        tokens = np.asarray(tokens, dtype=np.int64)
        tok_ad = w.token_adapter()[tokens]
        x = x[tokens]
        y_in = None if y_in is None else y_in[tokens]
        starts = np.arange(len(tokens) + 1, dtype=np.int32)
        segs = tok_ad.astype(np.int32)
    used = sorted({int(a) for a in segs if a >= 0})
    adapters = {}
    for a in used:
        A, B = w.adapter_block(a, layer, p)
        adapters[a] = (A, B, float(w.scales[a]))
    if not adapters and y_in is None:
        return np.zeros((x.shape[0], pr.h_out), np.float32 if acc == "f32" else np.float64)
    if w.sigma_kind:
        sig = w.seg_sigma
        if tokens is not None:
            row_sig = np.full(w.num_tokens, -1, np.int32)
            for si in range(w.num_segs):
                row_sig[w.seg_starts[si]:w.seg_starts[si + 1]] = sig[si]
            sig = row_sig[tokens]
        cores = np.stack([w.core(j, layer, p) for j in range(w.n_cores)])
        return lora_delta_sigma(x, starts, segs, sig, adapters, cores, w.sigma_kind, y_in,
                                acc=acc, threads=threads)
    return lora_delta(x, starts, segs, adapters, y_in, acc=acc, threads=threads)
