"""Seeded synthetic inputs for the MSA index-score operator.

This package only draws and lays out input tensors (queries, paged or packed
keys, int8 scales, block tables, sequence lengths, and score rows for the
top-k selection).  It holds none of the
operator's arithmetic, so both the CPU oracle's tests and the GPU path's tests
and benchmark can use it without sharing any scoring code.
"""
from .inputs import (  # noqa: F401
    MsaCase,
    CONFIG_NAMES,
    MX_CONFIG_NAMES,
    config_case,
    mx_config_case,
    e5m2_config_case,
    i8_prefill_config_case,
    make_case,
    edge_cases,
    random_cases,
    large_batch_cases,
    mx_random_cases,
    poison_case,
    case_summary,
    score_rows,
)
