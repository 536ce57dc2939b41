"""CPU oracle for decode attention over a KIVI-style asymmetric low-bit KV cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this package:
only the tests, the smoke check and the CPU-baseline leg of the benchmark use it.
It shares no code with the HIP library and imports nothing from it.
"""
from .kvq_oracle import (  # noqa: F401
    wht128_fp32,
    quantize_uniform,
    quantize_key_group,
    quantize_value_group,
    pack_group_block,
    unpack_group_block,
    dequantize_block,
    quantized_count,
    attention_fp64,
    rope_fp64,
    OracleHead,
    OracleCache,
    group_block_bytes,
)
