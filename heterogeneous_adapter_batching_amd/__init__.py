"""MI355X (gfx950) multi-adapter LoRA delta: Python binding of libhab_lora.so.

The library computes y[t] (+)= s_i * B_i (A_i x[t]) for a heterogeneous batch
whose token segments name adapters of an HBM-resident pool (the C ABI is
declared in include/lora_sgmv.h).  This module only marshals arguments:
torch tensors provide device memory and streams, and every step of the delta
runs in the library's HIP kernels.  There is no fallback: if the library is
missing or fails to load, importing the binding's entry points raises.
"""
from __future__ import annotations

from ._lib import (  # noqa: F401
    LIB_PATH, LoraError, PlanOpts, PoolDesc, load, status_name, LORA_F32, LORA_BF16,
    LORA_MAX_PROJ, LORA_MAX_RANK, LORA_SIGMA_DIAG, LORA_SIGMA_FULL, LORA_DEBUG_SLAB,
    LORA_DEBUG_TOKEN, LORA_DEBUG_ROW,
)
from .api import (  # noqa: F401
    Pool, Plan, sgmv_shrink, sgmv_expand, sgmv_fused, sgmv_expand_sigma, sgmv_fused_sigma,
    pool_bytes_for, extent_bytes, pack_adapter, Cache, sgmv_shrink_partials,
    sgmv_expand_partials, sgmv_expand_partials_sigma, sgmv_fused_static, plan_opts_default,
    debug_checks,
)

__all__ = ["Pool", "Plan", "sgmv_shrink", "sgmv_expand", "sgmv_fused", "sgmv_expand_sigma",
           "sgmv_fused_sigma", "sgmv_shrink_partials", "sgmv_expand_partials",
           "sgmv_expand_partials_sigma", "sgmv_fused_static",
           "pool_bytes_for", "extent_bytes", "pack_adapter", "Cache", "LoraError", "load",
           "plan_opts_default", "debug_checks"]
