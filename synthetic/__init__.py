"""Seeded synthetic inputs for the DSpark proposal step.

This package only draws random tensors and arranges them in the layouts the
library and the oracle both take. It holds none of the method's arithmetic
(no projection, no Markov bias, no argmax, no sigmoid): both the GPU path and
the CPU oracle consume what it returns, and neither is imported here.
"""
from .inputs import (  # noqa: F401
    CONFIGS,
    MASK_TOKEN_ID,
    Config,
    Inputs,
    Q4Inputs,
    ReducedInputs,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_inputs,
    make_small,
    q4_blocks,
    quantize_q4,
    reduce_vocab,
)
