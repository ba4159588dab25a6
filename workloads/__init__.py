"""Seeded synthetic inputs shared by the oracle's tests, the GPU parity tests
and the benchmark.

This package draws random numbers and lays out plain data (document ids,
bf16 tensors, per-head slopes). It performs none of the attention method's
arithmetic: no predicate, no tile classification, no softmax.
"""
from .generators import (  # noqa: F401
    MaskSpecData,
    ScoreModData,
    Workload,
    doc_ids_from_eot_flags,
    doc_ids_geometric,
    doc_ids_lognormal,
    doc_ids_chunks,
    random_bf16,
    random_f16,
    alibi_slopes,
    bias_table,
    make_config,
    CONFIG_NAMES,
)
