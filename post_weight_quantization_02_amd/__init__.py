"""GPTQ one-layer quantize-and-compensate on MI355X (gfx950).

The compute path is the HIP library libgptq_mi355x.so behind the C ABI in
include/gptq.h; this package is its Python binding. Importing it without the
built library raises ImportError.
"""
from ._lib import (  # noqa: F401
    GPTQError,
    GPTQ_DTYPE_F16,
    GPTQ_DTYPE_F32,
    GPTQ_ERR_HIP,
    GPTQ_ERR_INVALID_ARG,
    GPTQ_ERR_NOT_PD,
    GPTQ_ERR_UNSUPPORTED,
    GPTQ_ERR_WORKSPACE,
    GPTQ_OK,
    LIB_PATH,
    OP_ACCUMULATE,
    OP_PREPARE,
    OP_QUANTIZE,
    OP_QUANTIZE_PERM,
    act_order,
    dequant_gemm,
    hessian_accumulate,
    hessian_accumulate_noalloc,
    lib,
    linear_forward,
    pack_codes,
    packed_words,
    prepare_hinv,
    prepare_hinv_perm,
    prepare_hinv_three_step,
    quantize_layer,
    quantize_layer_perm,
    status_string,
    version,
    workspace_bytes,
)
from .pipeline import quantize_relu_block  # noqa: F401,E402
from .block import BlockLayer, BlockStream, quantize_streams  # noqa: F401,E402
