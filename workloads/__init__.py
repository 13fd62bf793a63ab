"""Seeded synthetic workloads (inputs only) and algorithmic byte/FLOP counts."""

from .synth import (  # noqa: F401
    PagedInputs,
    build_inputs,
    config_c1,
    config_c2,
    config_c3,
    config_c4,
    config_c5,
    make_config,
    CONFIGS,
    small_decode,
    small_extend,
    random_bf16,
    f32_to_bf16_bits,
    normal_bf16_stream,
)
from . import metrics  # noqa: F401
