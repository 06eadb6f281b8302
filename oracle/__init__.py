"""Plain fp64 CPU oracle for GPTQ's one-layer quantize-and-compensate path.

TEST INFRASTRUCTURE. Only the test-suite, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product path (the HIP library
and its Python binding) never imports, calls or falls back to it, and this
package imports nothing from the product path.
"""
from .gptq64 import (  # noqa: F401
    NotPositiveDefinite,
    hessian,
    damp,
    cholesky_lower,
    inverse_from_cholesky,
    hinv_upper,
    group_params,
    quantize,
    gptq,
    rtn,
    dequantize,
    output_error,
    layer_objective,
    act_order_perm,
    gptq_act_order,
    dequantize_gidx,
)
from .infer64 import (  # noqa: F401
    codes_per_word,
    pack_codes,
    unpack_codes,
    dequant_weights,
    dequant_matmul,
    abs_products,
)
from .pipeline64 import (  # noqa: F401
    quantize_one_layer,
    relu_to_f16,
    quantized_layer_output,
    two_layer_block,
)
