"""GPTQ layer-wise weight quantization solver for AMD Instinct MI355X (gfx950).

The solver's steps are HIP kernels behind a C ABI (include/gptq.h, libgptq.so); this package is its
Python binding. Build the library with `python -m post_weight_quantization_20_amd.build`.
"""

from .solver import (  # noqa: F401
    BLOCK_LAYERS,
    GPTQ_BF16,
    GPTQ_EHIP,
    GPTQ_EINVAL,
    GPTQ_ENOMEM,
    GPTQ_ENOTPD,
    GPTQ_EUNSUPPORTED,
    GPTQ_F16,
    GPTQ_F32,
    GPTQ_FACTOR_NOALLOC_MAX_D,
    GPTQ_LAYOUT_DENSE,
    GPTQ_LAYOUT_FIELDS,
    GPTQ_OK,
    GPTQ_WS_FACTOR,
    GPTQ_WS_HESSIAN,
    GPTQ_WS_QUANTIZE,
    BlockResult,
    BlockShape,
    GPTQError,
    LayerResult,
    Params,
    QuantOutput,
    gptq_block_workspace_bytes,
    gptq_dequant_gemm,
    gptq_factor,
    gptq_factor_noalloc,
    gptq_hessian_accumulate,
    gptq_pack,
    gptq_pack_dense,
    gptq_pack_ordered,
    gptq_permute_columns,
    packed_words,
    gptq_quantize_block,
    gptq_quantize_layer,
    gptq_workspace_bytes,
    quantize_layer,
)
