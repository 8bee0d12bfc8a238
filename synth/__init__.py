"""Seeded synthetic inputs shared by the oracle checks, the GPU tests and the bench.

This package only draws random numbers and lays them out in the storage formats the
library consumes (bf16 bit patterns, packed int4 bytes, fp32 scales). It holds none of
the method's arithmetic: no quantisation, routing, GEMM or combine happens here.
"""

from .inputs import (  # noqa: F401
    CONFIGS,
    MoEConfig,
    DenseConfig,
    StackConfig,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    moe_inputs,
    dense_inputs,
    stack_inputs,
    rng_for,
)
