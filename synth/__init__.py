"""Seeded synthetic inputs shared by the CPU oracle tests and the GPU path."""
from .workloads import (  # noqa: F401
    Proj, Workload, bf16_round, bf16_bits, bf16_to_f32, config, CONFIGS,
    random_case, zipf_probs, default_threads, MISTRAL_PROJS, jd_case, jd_full_stack,
    sweep_stack, sweep_assignments, mixed_case, merge_full_stack,
)
