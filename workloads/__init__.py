"""Seeded synthetic inputs for MLA decode over a paged KV cache.

This module only draws random numbers and lays them out in the shapes the
decode call takes; it holds none of the attention arithmetic.  Both the fp64
oracle and the HIP path consume the exact bytes produced here.
"""
from .mla_inputs import (  # noqa: F401
    CONFIGS,
    Workload,
    bf16_bits_from_f32,
    fp8_query,
    make_config,
    make_workload,
    batch_share,
    repage,
)
