"""Pool, Plan and the three sgmv calls over the C ABI (argument marshalling only)."""
from __future__ import annotations

import ctypes
import functools
from typing import Optional, Sequence

import numpy as np

from ._lib import (LORA_BF16, LORA_F32, LORA_MAX_PROJ, LORA_SIGMA_DIAG, LORA_SIGMA_FULL, PlanOpts,
                   PoolDesc, check, load)

_DTYPES = {"bf16": LORA_BF16, "f32": LORA_F32}


def _torch():
    import torch
    return torch


_TORCH_DTYPES = {}


def _torch_dtype(dtype: str):
    if dtype not in _TORCH_DTYPES:
        torch = _torch()
        _TORCH_DTYPES[dtype] = torch.bfloat16 if dtype == "bf16" else torch.float32
    return _TORCH_DTYPES[dtype]


def _stream_handle(stream) -> int:
    """The hipStream_t of a torch stream (the current one for None), as the
    integer the c_void_p arguments take."""
    if stream is None:
        stream = _torch().cuda.current_stream()
    return stream.cuda_stream


def _i32_array(values) -> ctypes.Array:
    vals = [int(v) for v in values]
    return (ctypes.c_int32 * max(len(vals), 1))(*vals)


@functools.lru_cache(maxsize=256)
def _i32_const(values: tuple) -> ctypes.Array:
    """A read-only int32 argument array, built once per distinct tuple: the
    per-call projection and y-offset lists of the sgmv calls (the library
    only reads them)."""
    return _i32_array(values)


def make_desc(num_layers: int, h_in: Sequence[int], h_out: Sequence[int], r_max: int,
              dtype: str = "bf16", max_slots: int = 1024, rank_granule: int = 8) -> PoolDesc:
    if len(h_in) != len(h_out) or not 1 <= len(h_in) <= LORA_MAX_PROJ:
        raise ValueError("h_in / h_out must list 1..8 projections")
    d = PoolDesc()
    d.num_layers = num_layers
    d.num_proj = len(h_in)
    for i, (a, b) in enumerate(zip(h_in, h_out)):
        d.h_in[i] = a
        d.h_out[i] = b
    d.r_max = r_max
    d.rank_granule = rank_granule
    d.max_slots = max_slots
    d.dtype = _DTYPES[dtype]
    return d


def pool_bytes_for(desc: PoolDesc, rank: int) -> int:
    """Bytes of one adapter at its true rank (no device needed)."""
    return int(load().lora_pool_bytes_for(ctypes.byref(desc), rank))


def extent_bytes(desc: PoolDesc, rank: int) -> int:
    """Bytes one adapter occupies in the slab (padded rank, 256-byte rounded)."""
    return int(load().lora_pool_extent_bytes(ctypes.byref(desc), rank))


def pack_adapter(desc: PoolDesc, rank: int, A: Sequence, B: Sequence, out=None) -> np.ndarray:
    """The packed extent image of one adapter (host, no device call): A[p]
    [L][rank][h_in_p], B[p] [L][h_out_p][rank] as host arrays of the pool
    dtype (float32, or uint16 bf16 bits).  `out`: a writable host buffer of at
    least extent_bytes(desc, rank) bytes (e.g. a pinned uint8 tensor's numpy
    view); a new uint8 array otherwise."""
    lib = load()
    n = extent_bytes(desc, rank)
    if out is None:
        out = np.empty(n, np.uint8)
    keep = [np.ascontiguousarray(a) for a in A] + [np.ascontiguousarray(b) for b in B]
    np_ = desc.num_proj
    arr_a = (ctypes.c_void_p * np_)(*[k.ctypes.data for k in keep[:np_]])
    arr_b = (ctypes.c_void_p * np_)(*[k.ctypes.data for k in keep[np_:]])
    ptr = out.ctypes.data if isinstance(out, np.ndarray) else out.data_ptr()
    nbytes = out.nbytes if isinstance(out, np.ndarray) else out.numel() * out.element_size()
    check(lib.lora_pack_adapter(ctypes.byref(desc), rank, arr_a, arr_b, ctypes.c_void_p(ptr),
                                nbytes))
    return out


def _check_dev(t, name, dtype=None, ndim=2):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim == 2 and t.numel() > 0 and t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} rows must be contiguous")


class Pool:
    """An adapter pool over one HBM slab.

    Either give ``slab`` (a CUDA tensor the pool will use; the caller keeps it
    alive) or ``slab_bytes`` (a uint8 CUDA tensor is allocated here).
    ``slab_ptr`` (an integer address) creates a host-metadata-only pool whose
    slab is never touched; it is for planning without a GPU.
    """

    def __init__(self, num_layers: int, h_in: Sequence[int], h_out: Sequence[int], r_max: int,
                 dtype: str = "bf16", max_slots: int = 1024, rank_granule: int = 8,
                 slab=None, slab_bytes: Optional[int] = None, slab_ptr: Optional[int] = None,
                 device: str = "cuda"):
        self.lib = load()
        self.desc = make_desc(num_layers, h_in, h_out, r_max, dtype, max_slots, rank_granule)
        self.dtype = dtype
        self.num_layers, self.h_in, self.h_out = num_layers, list(h_in), list(h_out)
        self.r_max = r_max
        self.slab = None
        if slab_ptr is not None:
            ptr, nbytes = slab_ptr, int(slab_bytes or 0)
        else:
            torch = _torch()
            if slab is None:
                if slab_bytes is None:
                    raise ValueError("give slab, slab_bytes or slab_ptr")
                slab = torch.empty(int(slab_bytes), dtype=torch.uint8, device=device)
            self.slab = slab
            ptr, nbytes = slab.data_ptr(), slab.numel() * slab.element_size()
        self._h = ctypes.c_void_p()
        check(self.lib.lora_pool_create(ctypes.byref(self._h), ctypes.byref(self.desc),
                                        ctypes.c_void_p(ptr), nbytes))

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            self.lib.lora_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    def extent_bytes(self, rank: int) -> int:
        return extent_bytes(self.desc, rank)

    def pool_bytes_for(self, rank: int) -> int:
        return pool_bytes_for(self.desc, rank)

    def plan_opts(self) -> dict:
        """The plan options plans built from this pool take (lora_plan_opts)."""
        o = PlanOpts()
        check(self.lib.lora_pool_get_plan_opts(self._h, ctypes.byref(o)))
        return _opts_dict(o)

    def set_plan_opts(self, **opts):
        """Set some of long_group, long_batch, shrink_groups, prefill_groups
        for plans built afterwards; the others keep their current values."""
        o = PlanOpts()
        check(self.lib.lora_pool_get_plan_opts(self._h, ctypes.byref(o)))
        for k, v in opts.items():
            if k not in _OPT_FIELDS:
                raise ValueError(f"unknown plan option {k!r}")
            setattr(o, k, int(v))
        check(self.lib.lora_pool_set_plan_opts(self._h, ctypes.byref(o)))

    def workspace_bytes(self, num_tokens: int, num_segs: int, max_proj: int = 3) -> int:
        """A workspace size that serves every plan of up to num_tokens tokens
        and num_segs segments over this pool."""
        return int(self.lib.lora_workspace_bytes(self._h, num_tokens, num_segs, max_proj))

    def reserve(self, adapter_id: int, rank: int, scale: float):
        check(self.lib.lora_pool_reserve(self._h, adapter_id, rank, ctypes.c_float(scale)))

    def upload(self, adapter_id: int, layer: int, proj: int, A, B, stream=None):
        """A: [rank][h_in], B: [h_out][rank], CUDA tensors of the pool dtype or
        host numpy arrays (float32 values for an f32 pool, uint16 bf16 bits
        for a bf16 pool)."""
        on_host = isinstance(A, np.ndarray)
        if on_host:
            A, B = np.ascontiguousarray(A), np.ascontiguousarray(B)
            pa, pb = A.ctypes.data, B.ctypes.data
        else:
            A, B = A.contiguous(), B.contiguous()
            pa, pb = A.data_ptr(), B.data_ptr()
        check(self.lib.lora_pool_upload(self._h, adapter_id, layer, proj, ctypes.c_void_p(pa),
                                        ctypes.c_void_p(pb), int(on_host), _stream_handle(stream)))

    def register(self, adapter_id: int, rank: int, scale: float, A: Sequence, B: Sequence,
                 stream=None):
        """A[p]: [L][rank][h_in_p], B[p]: [L][h_out_p][rank] for every projection,
        all CUDA tensors or all host numpy arrays (see ``upload``)."""
        on_host = isinstance(A[0], np.ndarray)
        keep = []
        ptrs_a, ptrs_b = [], []
        for a, b in zip(A, B):
            if on_host:
                a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
                ptrs_a.append(a.ctypes.data)
                ptrs_b.append(b.ctypes.data)
            else:
                a, b = a.contiguous(), b.contiguous()
                ptrs_a.append(a.data_ptr())
                ptrs_b.append(b.data_ptr())
            keep += [a, b]
        arr_a = (ctypes.c_void_p * len(ptrs_a))(*ptrs_a)
        arr_b = (ctypes.c_void_p * len(ptrs_b))(*ptrs_b)
        check(self.lib.lora_pool_register(self._h, adapter_id, rank, ctypes.c_float(scale),
                                          arr_a, arr_b, int(on_host), _stream_handle(stream)))

    def unregister(self, adapter_id: int):
        check(self.lib.lora_pool_unregister(self._h, adapter_id))

    def register_image(self, adapter_id: int, rank: int, scale: float, image, stream=None):
        """Reserve and copy a packed image (``pack_adapter``): a host numpy
        array or CPU tensor (pinned for an asynchronous copy), or a CUDA
        tensor.  The image must stay alive until the stream passes the copy."""
        ptr, on_host = _image_ptr(image)
        check(self.lib.lora_pool_register_image(self._h, adapter_id, rank, ctypes.c_float(scale),
                                                ctypes.c_void_p(ptr), int(on_host),
                                                _stream_handle(stream)))

    def query(self, adapter_id: int):
        r, rp = ctypes.c_int32(), ctypes.c_int32()
        sc, off = ctypes.c_float(), ctypes.c_uint64()
        check(self.lib.lora_pool_query(self._h, adapter_id, ctypes.byref(r), ctypes.byref(rp),
                                       ctypes.byref(sc), ctypes.byref(off)))
        return {"rank": r.value, "r_pad": rp.value, "scale": sc.value, "offset": off.value}

    def stats(self):
        n, free = ctypes.c_int32(), ctypes.c_uint64()
        check(self.lib.lora_pool_stats(self._h, ctypes.byref(n), ctypes.byref(free)))
        return {"adapters": n.value, "free_bytes": free.value}


def _image_ptr(image):
    if isinstance(image, np.ndarray):
        return image.ctypes.data, True
    return image.data_ptr(), not image.is_cuda


class Cache:
    """Adapter exchange over a pool: host-resident packed adapters made
    resident on demand on a copy stream, least recently used evicted (see
    lora_cache_* in the C header).  Images are kept referenced here."""

    def __init__(self, pool: Pool, copy_stream=None):
        torch = _torch()
        self.lib = pool.lib
        self.pool = pool
        self.copy_stream = copy_stream if copy_stream is not None else torch.cuda.Stream()
        self._images = {}
        self._h = ctypes.c_void_p()
        check(self.lib.lora_cache_create(ctypes.byref(self._h), pool.handle,
                                         ctypes.c_void_p(self.copy_stream.cuda_stream)))

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            self.lib.lora_cache_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add(self, adapter_id: int, rank: int, scale: float, image):
        ptr, on_host = _image_ptr(image)
        if not on_host:
            raise ValueError("cache images live in host memory")
        check(self.lib.lora_cache_add(self._h, adapter_id, rank, ctypes.c_float(scale),
                                      ctypes.c_void_p(ptr)))
        self._images[adapter_id] = image

    def acquire(self, ids, stream=None) -> int:
        arr = _i32_array(ids)
        up = ctypes.c_int32()
        check(self.lib.lora_cache_acquire(self._h, len(list(ids)), arr, _stream_handle(stream),
                                          ctypes.byref(up)))
        return up.value

    def release(self, stream=None):
        check(self.lib.lora_cache_release(self._h, _stream_handle(stream)))

    def prefetch(self, ids) -> int:
        arr = _i32_array(ids)
        up = ctypes.c_int32()
        check(self.lib.lora_cache_prefetch(self._h, len(list(ids)), arr, ctypes.byref(up)))
        return up.value

    def query(self, adapter_id: int):
        r, h = ctypes.c_int32(), ctypes.c_int32()
        check(self.lib.lora_cache_query(self._h, adapter_id, ctypes.byref(r), ctypes.byref(h)))
        return {"resident": bool(r.value), "held": bool(h.value)}

    def stats(self):
        n = ctypes.c_int32()
        v = [ctypes.c_uint64() for _ in range(5)]
        check(self.lib.lora_cache_stats(self._h, ctypes.byref(n), *[ctypes.byref(x) for x in v]))
        return dict(zip(("resident", "hits", "misses", "prefetched", "evictions",
                         "bytes_uploaded"), [n.value] + [x.value for x in v]))


class Plan:
    """The gather plan of one heterogeneous batch (built on the host)."""

    def __init__(self, pool: Pool, num_tokens: int, seg_starts, seg_adapter, seg_sigma=None,
                 seg_weight=None):
        """seg_sigma: per-segment core index of jointly compressed adapters
        (-1: none), or None for plain adapters.  seg_weight: per-segment
        weight that scales each token's delta (one slot of a weighted merge),
        or None."""
        self.lib = pool.lib
        self.pool = pool
        self.num_tokens = int(num_tokens)
        starts = np.ascontiguousarray(seg_starts, dtype=np.int32)
        segs = np.ascontiguousarray(seg_adapter, dtype=np.int32)
        if starts.ndim != 1 or segs.ndim != 1 or starts.shape[0] != segs.shape[0] + 1:
            raise ValueError("seg_starts must have one more entry than seg_adapter")
        self._h = ctypes.c_void_p()
        i32p = ctypes.POINTER(ctypes.c_int32)
        if seg_sigma is not None and seg_weight is not None:
            raise ValueError("a plan takes cores or weights, not both")
        if seg_weight is not None:
            wts = np.ascontiguousarray(seg_weight, dtype=np.float32)
            if wts.shape != segs.shape:
                raise ValueError("seg_weight must have one entry per segment")
            check(self.lib.lora_plan_create_weighted(
                ctypes.byref(self._h), pool.handle, self.num_tokens, starts.ctypes.data_as(i32p),
                segs.ctypes.data_as(i32p), wts.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                int(segs.shape[0])))
        elif seg_sigma is None:
            check(self.lib.lora_plan_create(ctypes.byref(self._h), pool.handle, self.num_tokens,
                                            starts.ctypes.data_as(i32p),
                                            segs.ctypes.data_as(i32p), int(segs.shape[0])))
        else:
            sig = np.ascontiguousarray(seg_sigma, dtype=np.int32)
            if sig.shape != segs.shape:
                raise ValueError("seg_sigma must have one entry per segment")
            check(self.lib.lora_plan_create_sigma(ctypes.byref(self._h), pool.handle,
                                                  self.num_tokens, starts.ctypes.data_as(i32p),
                                                  segs.ctypes.data_as(i32p),
                                                  sig.ctypes.data_as(i32p), int(segs.shape[0])))
        self.ws = None
        self.max_proj = 0

    @classmethod
    def merge(cls, pool: Pool, num_tokens: int, seg_starts, seg_adapters, seg_weights):
        """A weighted merge of K adapters per request: seg_adapters and
        seg_weights are [S][K] (adapter -1: an empty slot).  sgmv_fused with
        this plan adds sum_k (w_k s_k) B_k (A_k x) in one pass."""
        starts = np.ascontiguousarray(seg_starts, dtype=np.int32)
        ads = np.ascontiguousarray(seg_adapters, dtype=np.int32)
        wts = np.ascontiguousarray(seg_weights, dtype=np.float32)
        if ads.ndim != 2 or wts.shape != ads.shape or starts.shape[0] != ads.shape[0] + 1:
            raise ValueError("seg_adapters and seg_weights must be [S][K], seg_starts [S+1]")
        self = cls.__new__(cls)
        self.lib = pool.lib
        self.pool = pool
        self.num_tokens = int(num_tokens)
        self._h = ctypes.c_void_p()
        i32p = ctypes.POINTER(ctypes.c_int32)
        check(self.lib.lora_plan_create_merge(
            ctypes.byref(self._h), pool.handle, self.num_tokens, starts.ctypes.data_as(i32p),
            int(ads.shape[0]), int(ads.shape[1]), ads.ctypes.data_as(i32p),
            wts.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))
        self.ws = None
        self.max_proj = 0
        return self

    def rebuild(self, num_tokens: int, seg_starts, seg_adapter, seg_sigma=None, seg_weight=None):
        """Re-plan for the next batch over the same pool, in place (host
        tables and pinned staging reused); upload again before the next call."""
        starts = np.ascontiguousarray(seg_starts, dtype=np.int32)
        segs = np.ascontiguousarray(seg_adapter, dtype=np.int32)
        if starts.ndim != 1 or segs.ndim != 1 or starts.shape[0] != segs.shape[0] + 1:
            raise ValueError("seg_starts must have one more entry than seg_adapter")
        i32p = ctypes.POINTER(ctypes.c_int32)
        sig = None if seg_sigma is None else np.ascontiguousarray(seg_sigma, dtype=np.int32)
        wts = None if seg_weight is None else np.ascontiguousarray(seg_weight, dtype=np.float32)
        for a, name in ((sig, "seg_sigma"), (wts, "seg_weight")):
            if a is not None and a.shape != segs.shape:
                raise ValueError(f"{name} must have one entry per segment")
        check(self.lib.lora_plan_rebuild(
            self._h, int(num_tokens), starts.ctypes.data_as(i32p), segs.ctypes.data_as(i32p),
            sig.ctypes.data_as(i32p) if sig is not None else None,
            wts.ctypes.data_as(ctypes.POINTER(ctypes.c_float)) if wts is not None else None,
            int(segs.shape[0])))
        self.num_tokens = int(num_tokens)
        return self

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            self.lib.lora_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    def workspace_bytes(self, max_proj: int) -> int:
        return int(self.lib.lora_plan_workspace_bytes(self._h, max_proj))

    def upload(self, max_proj: int = 3, ws=None, stream=None):
        """Copy the plan into a device workspace (allocated here unless given)."""
        torch = _torch()
        need = self.workspace_bytes(max_proj)
        if ws is None:
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        check(self.lib.lora_plan_upload(self._h, ctypes.c_void_p(ws.data_ptr()),
                                        ws.numel() * ws.element_size(), max_proj,
                                        _stream_handle(stream)))
        self.ws = ws
        self.max_proj = max_proj
        return self

    def stats(self):
        vals = [ctypes.c_int32() for _ in range(4)]
        check(self.lib.lora_plan_stats(self._h, *[ctypes.byref(v) for v in vals]))
        return dict(zip(("groups", "blocks", "active_tokens", "max_block_tokens"),
                        [v.value for v in vals]))

    def opts(self) -> dict:
        """The plan options this plan was built with (its pool's at the time)."""
        o = PlanOpts()
        check(self.lib.lora_plan_get_opts(self._h, ctypes.byref(o)))
        return _opts_dict(o)

    def export(self):
        st = self.stats()
        T, G = self.num_tokens, st["groups"]
        order = np.zeros(max(T, 1), np.int32)
        tgroup = np.zeros(max(T, 1), np.int32)
        gad = np.zeros(max(G, 1), np.int32)
        grank = np.zeros(max(G, 1), np.int32)
        i32p = ctypes.POINTER(ctypes.c_int32)
        check(self.lib.lora_plan_export(self._h, order.ctypes.data_as(i32p),
                                        tgroup.ctypes.data_as(i32p), gad.ctypes.data_as(i32p),
                                        grank.ctypes.data_as(i32p)))
        return {"token_order": order[:T], "token_group": tgroup[:T],
                "group_adapter": gad[:G], "group_rank": grank[:G]}


_OPT_FIELDS = tuple(f[0] for f in PlanOpts._fields_)


def _opts_dict(o) -> dict:
    return {k: int(getattr(o, k)) for k in _OPT_FIELDS}


def plan_opts_default() -> dict:
    """The library's default plan options."""
    o = PlanOpts()
    load().lora_plan_opts_default(ctypes.byref(o))
    return _opts_dict(o)


def debug_checks(clear: bool = False):
    """(enabled, errors): whether the loaded library is the bounds-checked
    debug build, and the LORA_DEBUG_* bits its kernels set on the current
    device since the last clear (waits for the device; 0 in the release
    build); `clear` resets them."""
    en, bits = ctypes.c_int32(), ctypes.c_uint32()
    check(load().lora_debug_checks(ctypes.byref(en), ctypes.byref(bits), int(bool(clear))))
    return bool(en.value), int(bits.value)


def _projs(projs):
    t = tuple(int(p) for p in projs)
    return len(t), _i32_const(t)


def _offsets(y_offsets):
    return _i32_const(tuple(int(o) for o in y_offsets))


def sgmv_shrink(pool: Pool, plan: Plan, layer: int, projs, x, v=None, stream=None):
    """v[:, i*r_max : i*r_max + r_max] = A_i,p x for each listed projection."""
    torch = _torch()
    _check_dev(x, "x", _torch_dtype(pool.dtype))
    n, parr = _projs(projs)
    if v is None:
        v = torch.zeros((x.shape[0], n * pool.r_max), dtype=torch.float32, device=x.device)
    _check_dev(v, "v", torch.float32)
    check(pool.lib.sgmv_shrink(pool.handle, plan.handle, layer, n, parr,
                               x.data_ptr(), x.stride(0),
                               v.data_ptr(), v.stride(0),
                               _stream_handle(stream)))
    return v


def sgmv_expand(pool: Pool, plan: Plan, layer: int, projs, y_offsets, v, y, stream=None):
    """y[:, off_i : off_i + h_out] += s * B_i,p v_i (rounded once)."""
    torch = _torch()
    _check_dev(v, "v", torch.float32)
    _check_dev(y, "y", _torch_dtype(pool.dtype))
    n, parr = _projs(projs)
    check(pool.lib.sgmv_expand(pool.handle, plan.handle, layer, n, parr, _offsets(y_offsets),
                               v.data_ptr(), v.stride(0),
                               y.data_ptr(), y.stride(0),
                               _stream_handle(stream)))
    return y


def sgmv_fused(pool: Pool, plan: Plan, layer: int, projs, y_offsets, x, y, base=None,
               stream=None):
    """y = (base or y) + s * B (A x) for each listed projection's slice of y."""
    dt = _torch_dtype(pool.dtype)
    _check_dev(x, "x", dt)
    _check_dev(y, "y", dt)
    if base is not None:
        _check_dev(base, "base", dt)
    n, parr = _projs(projs)
    check(pool.lib.sgmv_fused(pool.handle, plan.handle, layer, n, parr, _offsets(y_offsets),
                              x.data_ptr(), x.stride(0),
                              (base.data_ptr() if base is not None else 0),
                              base.stride(0) if base is not None else 0,
                              y.data_ptr(), y.stride(0),
                              _stream_handle(stream)))
    return y


def sgmv_fused_static(pool: Pool, plan: Plan, layer: int, projs, y_offsets, x, y, base=None,
                      stream=None):
    """sgmv_fused with the shrink partials in the library's static device
    scratch: the call allocates nothing.  Calls on one GPU must not overlap."""
    dt = _torch_dtype(pool.dtype)
    _check_dev(x, "x", dt)
    _check_dev(y, "y", dt)
    if base is not None:
        _check_dev(base, "base", dt)
    n, parr = _projs(projs)
    check(pool.lib.sgmv_fused_static(pool.handle, plan.handle, layer, n, parr,
                                     _offsets(y_offsets),
                                     x.data_ptr(), x.stride(0),
                                     (base.data_ptr() if base is not None else 0),
                                     base.stride(0) if base is not None else 0,
                                     y.data_ptr(), y.stride(0),
                                     _stream_handle(stream)))
    return y


def sgmv_shrink_partials(pool: Pool, plan: Plan, layer: int, projs, x, stream=None):
    """The shrink of sgmv_fused alone: partial sums of v = A x left in the
    plan's workspace for sgmv_expand_partials of the same call."""
    _check_dev(x, "x", _torch_dtype(pool.dtype))
    n, parr = _projs(projs)
    check(pool.lib.sgmv_shrink_partials(pool.handle, plan.handle, layer, n, parr,
                                        x.data_ptr(), x.stride(0),
                                        _stream_handle(stream)))


def sgmv_expand_partials(pool: Pool, plan: Plan, layer: int, projs, y_offsets, y, base=None,
                         stream=None):
    """The expand of sgmv_fused alone, from the partials of the plan's last
    shrink (which must be this call's): y = (base or y) + s * B v."""
    dt = _torch_dtype(pool.dtype)
    _check_dev(y, "y", dt)
    if base is not None:
        _check_dev(base, "base", dt)
    n, parr = _projs(projs)
    check(pool.lib.sgmv_expand_partials(pool.handle, plan.handle, layer, n, parr,
                                        _offsets(y_offsets),
                                        (base.data_ptr() if base is not None else 0),
                                        base.stride(0) if base is not None else 0,
                                        y.data_ptr(), y.stride(0),
                                        _stream_handle(stream)))
    return y


def sgmv_expand_partials_sigma(pool: Pool, plan: Plan, layer: int, projs, y_offsets, sigma, kind,
                               y, base=None, stream=None):
    """sgmv_expand_partials with the core step of jointly compressed adapters."""
    dt = _torch_dtype(pool.dtype)
    _check_dev(y, "y", dt)
    if base is not None:
        _check_dev(base, "base", dt)
    _check_cores(pool, sigma, kind)
    n, parr = _projs(projs)
    check(pool.lib.sgmv_expand_partials_sigma(
        pool.handle, plan.handle, layer, n, parr, _offsets(y_offsets),
        sigma.data_ptr(), _sigma_kind(kind), sigma.shape[0],
        (base.data_ptr() if base is not None else 0),
        base.stride(0) if base is not None else 0, y.data_ptr(), y.stride(0),
        _stream_handle(stream)))
    return y


def _sigma_kind(kind) -> int:
    codes = {"diag": LORA_SIGMA_DIAG, "full": LORA_SIGMA_FULL}
    if kind not in codes:
        raise ValueError(f"core kind {kind!r} is neither 'diag' nor 'full'")
    return codes[kind]


def _check_cores(pool: Pool, sigma, kind):
    torch = _torch()
    _check_dev(sigma, "sigma", torch.float32, ndim=sigma.dim() if hasattr(sigma, "dim") else 2)
    if not sigma.is_contiguous():
        raise ValueError("sigma must be contiguous")
    tail = (pool.num_layers, len(pool.h_in), pool.r_max) + ((pool.r_max,) if kind == "full" else ())
    if tuple(sigma.shape[1:]) != tail:
        raise ValueError(f"sigma must be [n]{list(tail)}, got {list(sigma.shape)}")
    return int(sigma.shape[0])


def sgmv_expand_sigma(pool: Pool, plan: Plan, layer: int, projs, y_offsets, v, sigma, kind, y,
                      stream=None):
    """y[:, off_i : off_i + h_out] += s * B_c,p (Sigma_k v_i): the B step of
    jointly compressed adapters after their core step.  sigma: float32
    [n][layers][proj][r_max][r_max] ("full") or [n][layers][proj][r_max] ("diag")."""
    torch = _torch()
    _check_dev(v, "v", torch.float32)
    _check_dev(y, "y", _torch_dtype(pool.dtype))
    n_sig = _check_cores(pool, sigma, kind)
    n, parr = _projs(projs)
    check(pool.lib.sgmv_expand_sigma(pool.handle, plan.handle, layer, n, parr,
                                     _offsets(y_offsets),
                                     v.data_ptr(), v.stride(0),
                                     sigma.data_ptr(), _sigma_kind(kind), n_sig,
                                     y.data_ptr(), y.stride(0),
                                     _stream_handle(stream)))
    return y


def sgmv_fused_sigma(pool: Pool, plan: Plan, layer: int, projs, y_offsets, x, sigma, kind, y,
                     base=None, stream=None):
    """y = (base or y) + s * B_c (Sigma_k (A_c x)) for each listed projection's
    slice of y: the three steps of jointly compressed adapters."""
    dt = _torch_dtype(pool.dtype)
    _check_dev(x, "x", dt)
    _check_dev(y, "y", dt)
    if base is not None:
        _check_dev(base, "base", dt)
    n_sig = _check_cores(pool, sigma, kind)
    n, parr = _projs(projs)
    check(pool.lib.sgmv_fused_sigma(pool.handle, plan.handle, layer, n, parr,
                                    _offsets(y_offsets),
                                    x.data_ptr(), x.stride(0),
                                    sigma.data_ptr(), _sigma_kind(kind), n_sig,
                                    (base.data_ptr() if base is not None else 0),
                                    base.stride(0) if base is not None else 0,
                                    y.data_ptr(), y.stride(0),
                                    _stream_handle(stream)))
    return y
