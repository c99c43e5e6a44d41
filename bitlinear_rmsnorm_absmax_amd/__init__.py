"""MI355X (gfx950) ternary BitLinear layer: Python binding of libbitlinear.so.

The C ABI is declared in include/bitlinear.h; this package only marshals torch
tensors (device memory, current stream) into those calls.
"""

from ._lib import (BF16, ERR_ALIGN, ERR_DTYPE, ERR_HIP, ERR_NULL, ERR_SHAPE, ERR_VALUE, F32,
                   MAX_K, OK, PATH_AUTO, PATH_GEMM, PATH_GEMV, PATH_SKINNY, BitLinearError,
                   abi_version, bitlinear, declared_symbols, forward, glu, last_error, lib,
                   pack_weights, quant_act, quant_forward, silu_mul_quant, silu_mul_quant_acc, ternarize, binarize,
                   pack_weights1, forward1, quant_act_grouped, forward_grouped,
                   ternarize_grouped, pack_weights3, forward3)

__all__ = ["quant_act", "pack_weights", "forward", "quant_forward", "silu_mul_quant", "silu_mul_quant_acc", "ternarize", "binarize",
           "pack_weights1", "forward1", "quant_act_grouped", "forward_grouped",
           "ternarize_grouped", "pack_weights3", "forward3", "bitlinear", "glu",
           "last_error", "abi_version", "declared_symbols", "lib", "BitLinearError"]
