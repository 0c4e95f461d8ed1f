"""ctypes declarations of the C ABI in include/lora_sgmv.h."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; HAB_LORA_LIB names another build of the same library to
# load instead (e.g. the sanitizer build of the host code the tests run).
LIB_PATH = os.environ.get("HAB_LORA_LIB") or os.path.join(PKG, "libhab_lora.so")

LORA_F32, LORA_BF16 = 0, 1
LORA_MAX_PROJ = 8
LORA_MAX_RANK = 64
LORA_STATIC_SCRATCH_MIB = 64
LORA_MAX_MERGE = 4
LORA_DEBUG_SLAB, LORA_DEBUG_TOKEN, LORA_DEBUG_ROW = 1, 2, 4

STATUS = {0: "LORA_OK", -1: "LORA_EINVAL", -2: "LORA_ENOSPC", -3: "LORA_ENOENT",
          -4: "LORA_ERANK", -5: "LORA_EDTYPE", -6: "LORA_ESEG", -7: "LORA_EHIP",
          -8: "LORA_EEXIST", -9: "LORA_ESTATE"}


def status_name(code: int) -> str:
    return STATUS.get(code, f"status {code}")


class LoraError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_name(status)}: {message}")
        self.status = status
        self.message = message


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_proj", ctypes.c_int32),
                ("h_in", ctypes.c_int32 * LORA_MAX_PROJ), ("h_out", ctypes.c_int32 * LORA_MAX_PROJ),
                ("r_max", ctypes.c_int32), ("rank_granule", ctypes.c_int32),
                ("max_slots", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class PlanOpts(ctypes.Structure):
    _fields_ = [("long_group", ctypes.c_int32), ("long_batch", ctypes.c_int32),
                ("shrink_groups", ctypes.c_int32), ("prefill_groups", ctypes.c_int32)]


_i32, _i64, _u64, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
_vp, _i32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)
_pp = ctypes.POINTER(ctypes.c_void_p)

# name: (restype, argtypes)
SIGNATURES = {
    "lora_last_error": (ctypes.c_char_p, []),
    "lora_pool_bytes_for": (_u64, [ctypes.POINTER(PoolDesc), _i32]),
    "lora_pool_extent_bytes": (_u64, [ctypes.POINTER(PoolDesc), _i32]),
    "lora_pool_create": (_i32, [ctypes.POINTER(_vp), ctypes.POINTER(PoolDesc), _vp, _u64]),
    "lora_pool_destroy": (_i32, [_vp]),
    "lora_pool_reserve": (_i32, [_vp, _i32, _i32, _f32]),
    "lora_pool_upload": (_i32, [_vp, _i32, _i32, _i32, _vp, _vp, _i32, _vp]),
    "lora_pool_register": (_i32, [_vp, _i32, _i32, _f32, _pp, _pp, _i32, _vp]),
    "lora_pool_unregister": (_i32, [_vp, _i32]),
    "lora_pool_query": (_i32, [_vp, _i32, _i32p, _i32p, ctypes.POINTER(_f32),
                               ctypes.POINTER(_u64)]),
    "lora_pool_stats": (_i32, [_vp, _i32p, ctypes.POINTER(_u64)]),
    "lora_plan_create": (_i32, [ctypes.POINTER(_vp), _vp, _i32, _i32p, _i32p, _i32]),
    "lora_plan_destroy": (_i32, [_vp]),
    "lora_plan_opts_default": (None, [ctypes.POINTER(PlanOpts)]),
    "lora_pool_set_plan_opts": (_i32, [_vp, ctypes.POINTER(PlanOpts)]),
    "lora_pool_get_plan_opts": (_i32, [_vp, ctypes.POINTER(PlanOpts)]),
    "lora_plan_get_opts": (_i32, [_vp, ctypes.POINTER(PlanOpts)]),
    "lora_debug_checks": (_i32, [_i32p, ctypes.POINTER(ctypes.c_uint32), _i32]),
    "lora_plan_workspace_bytes": (_u64, [_vp, _i32]),
    "lora_workspace_bytes": (_u64, [_vp, _i32, _i32, _i32]),
    "lora_plan_rebuild": (_i32, [_vp, _i32, _i32p, _i32p, _i32p, ctypes.POINTER(_f32), _i32]),
    "lora_plan_upload": (_i32, [_vp, _vp, _u64, _i32, _vp]),
    "lora_plan_stats": (_i32, [_vp, _i32p, _i32p, _i32p, _i32p]),
    "lora_plan_export": (_i32, [_vp, _i32p, _i32p, _i32p, _i32p]),
    "sgmv_shrink": (_i32, [_vp, _vp, _i32, _i32, _i32p, _vp, _i64, _vp, _i64, _vp]),
    "sgmv_expand": (_i32, [_vp, _vp, _i32, _i32, _i32p, _i32p, _vp, _i64, _vp, _i64, _vp]),
    "sgmv_fused": (_i32, [_vp, _vp, _i32, _i32, _i32p, _i32p, _vp, _i64, _vp, _i64, _vp, _i64,
                          _vp]),
    "lora_plan_create_sigma": (_i32, [ctypes.POINTER(_vp), _vp, _i32, _i32p, _i32p, _i32p, _i32]),
    "lora_plan_create_weighted": (_i32, [ctypes.POINTER(_vp), _vp, _i32, _i32p, _i32p,
                                         ctypes.POINTER(_f32), _i32]),
    "lora_plan_create_merge": (_i32, [ctypes.POINTER(_vp), _vp, _i32, _i32p, _i32, _i32, _i32p,
                                      ctypes.POINTER(_f32)]),
    "sgmv_expand_sigma": (_i32, [_vp, _vp, _i32, _i32, _i32p, _i32p, _vp, _i64, _vp, _i32, _i32,
                                 _vp, _i64, _vp]),
    "sgmv_fused_sigma": (_i32, [_vp, _vp, _i32, _i32, _i32p, _i32p, _vp, _i64, _vp, _i32, _i32,
                                _vp, _i64, _vp, _i64, _vp]),
    "sgmv_fused_static": (_i32, [_vp, _vp, _i32, _i32, _i32p, _i32p, _vp, _i64, _vp, _i64, _vp,
                                 _i64, _vp]),
    "sgmv_shrink_partials": (_i32, [_vp, _vp, _i32, _i32, _i32p, _vp, _i64, _vp]),
    "sgmv_expand_partials": (_i32, [_vp, _vp, _i32, _i32, _i32p, _i32p, _vp, _i64, _vp, _i64,
                                    _vp]),
    "sgmv_expand_partials_sigma": (_i32, [_vp, _vp, _i32, _i32, _i32p, _i32p, _vp, _i32, _i32,
                                          _vp, _i64, _vp, _i64, _vp]),
    "lora_pack_adapter": (_i32, [ctypes.POINTER(PoolDesc), _i32, _pp, _pp, _vp, _u64]),
    "lora_pool_upload_image": (_i32, [_vp, _i32, _vp, _i32, _vp]),
    "lora_pool_register_image": (_i32, [_vp, _i32, _i32, _f32, _vp, _i32, _vp]),
    "lora_pool_get_desc": (_i32, [_vp, ctypes.POINTER(PoolDesc)]),
    "lora_cache_create": (_i32, [ctypes.POINTER(_vp), _vp, _vp]),
    "lora_cache_destroy": (_i32, [_vp]),
    "lora_cache_add": (_i32, [_vp, _i32, _i32, _f32, _vp]),
    "lora_cache_acquire": (_i32, [_vp, _i32, _i32p, _vp, _i32p]),
    "lora_cache_release": (_i32, [_vp, _vp]),
    "lora_cache_prefetch": (_i32, [_vp, _i32, _i32p, _i32p]),
    "lora_cache_query": (_i32, [_vp, _i32, _i32p, _i32p]),
    "lora_cache_stats": (_i32, [_vp, _i32p, ctypes.POINTER(_u64), ctypes.POINTER(_u64),
                                ctypes.POINTER(_u64), ctypes.POINTER(_u64),
                                ctypes.POINTER(_u64)]),
}

LORA_SIGMA_DIAG, LORA_SIGMA_FULL = 1, 2

_lib = None


def load():
    """Load libhab_lora.so (built in-tree by __graft_entry__.build()).

    Raises ImportError when the library has not been built: there is no other
    implementation to fall back to."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int) -> None:
    if status != 0:
        msg = load().lora_last_error()
        raise LoraError(status, msg.decode() if msg else "")
