"""MI355X (gfx950) GPTQ layer quantizer: Hessian SYRK, damped inverse Cholesky
factor, lazy-block quantize-and-repair, int3/int4 packing, the dequantizing
matrix-vector product over the packed words and the Hadamard pre-rotation, as
hand-written HIP kernels behind the C ABI in include/gptq.h."""
from .gptq import (GPTQError, NotPositiveDefinite, Workspace, dequant_gemv, hadamard_rotate, hessian_accumulate,
                   pack, prepare, quantize_layer)

__all__ = ["hessian_accumulate", "prepare", "quantize_layer", "pack", "dequant_gemv", "hadamard_rotate", "Workspace",
           "NotPositiveDefinite", "GPTQError"]
