"""Seeded synthetic inputs for the wide-beam decode step.

This package is shared by the oracle side (tests, cpu baseline) and the GPU side
(tests, bench).  It produces inputs only: catalogs of semantic-ID items, the CSR
layout of their prefix trie, attention tensors in their storage formats, and
log-probability rows, raw logit rows, and the noise rows of the sampled selection.  It holds none of the attention or selection arithmetic.
"""
from .workloads import (  # noqa: F401
    Workload,
    WORKLOADS,
    workload,
    request_shapes,
    catalog_items,
    build_trie_csr,
    attention_layer,
    logprob_rows,
    gumbel_rows,
    logit_rows,
    random_parents,
    pack_prefix,
    bf16_bits_from_f32,
    e4m3fn_bits_from_f32,
)
