"""CPU oracle for Hybrid-Engine experience generation (test infrastructure).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import this package.  It shares no code
with the GPU library and imports nothing from it.
"""
from .opt_he import (  # noqa: F401
    Precision, round_bf16, round_fp32, lora_delta, lora_fuse, lora_unfuse,
    layer_norm, causal_attention, argmax_lowest, OracleModel, greedy_generate,
    ulp_bf16,
)
