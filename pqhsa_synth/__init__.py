"""Seeded synthetic inputs for PQ-HSA decode attention.

This package only draws random numbers and lays them out (bf16 rounding,
paging).  It computes nothing that the attention method computes; both the
oracle and the HIP path receive the arrays it produces.
"""
from .gen import (  # noqa: F401
    WORKLOADS,
    HeadDraw,
    StepInputs,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    make_query_stream,
    make_step_inputs,
    page_layout,
    to_paged,
)
