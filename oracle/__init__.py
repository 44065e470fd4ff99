"""Float64 CPU oracle for PQ-HSA decode attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; never by the product path.
"""
from .pqhsa_oracle import (  # noqa: F401
    approx_logits,
    bf16_to_f64,
    bruteforce_head_group,
    budget_k,
    cluster_means,
    decode_step,
    dense_attention,
    dense_step,
    head_group_step,
    lse_merge,
    lut_tables,
    partial_attention,
    partition,
    select_topk,
)
