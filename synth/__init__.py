"""Seeded synthetic inputs (weights and calibration activations) for the GPTQ layer solver."""

from .gen import (  # noqa: F401
    CONFIGS,
    LayerCase,
    Workload,
    bf16_bits_to_f64,
    case_from_config,
    make_case,
    outlier_channels,
    round_to_dtype,
    to_f64,
    weight,
    x_chunk,
    x_tokens,
)
