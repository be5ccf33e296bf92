"""Seeded synthetic inputs (weights and calibration activations) for the GPTQ layer solver."""

from .gen import (  # noqa: F401
    CONFIGS,
    BlockCase,
    LayerCase,
    StoredLayer,
    Workload,
    bf16_bits_to_f64,
    block_layer_dims,
    block_weights,
    block_x,
    case_from_config,
    inference_x,
    make_case,
    outlier_channels,
    round_to_dtype,
    stored_layer,
    to_f64,
    weight,
    x_chunk,
    x_tokens,
)
