"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the benchmark.

This package draws keys, values, window queries, page tables and budgets. It
holds none of the compression method's arithmetic (no scoring, no selection,
no compaction), so both sides of every parity check can take their inputs from
it without sharing any of the computation being checked.
"""
from .gen import (  # noqa: F401
    bf16_round,
    segment_layout,
    plant_near_duplicates,
    DenseCase,
    PagedCase,
    tiny_head_case,
    dense_case_host,
    dense_case_device,
    paged_case_host,
    paged_case_device,
    CONFIGS,
)
