"""fp64 CPU oracle for MLA decode over a paged KV cache -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library never calls it, and it shares no code,
headers, tables or helpers with the HIP path.
"""
from .mla_oracle import (  # noqa: F401
    E4M3FN_TABLE,
    attend,
    bf16_bits_to_f64,
    decode_kv,
    e4m3fn_code_to_f64,
    fused_fp8_scales,
    gather_rows,
    lse_merge,
    mla_decode,
    mla_decode_f64,
    visible_keys,
)
from .schedule_oracle import check_schedule, expand_splits, schedule  # noqa: F401
