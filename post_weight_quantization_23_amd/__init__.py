"""MI355X (gfx950) GPTQ layer quantizer: Hessian SYRK, damped inverse Cholesky
factor, lazy-block quantize-and-repair, int3/int4 packing and the
dequantizing matrix-vector product over the packed words, as hand-written HIP
kernels behind the C ABI in include/gptq.h."""
from .gptq import (GPTQError, NotPositiveDefinite, Workspace, dequant_gemv, hessian_accumulate, pack,
                   prepare, quantize_layer)

__all__ = ["hessian_accumulate", "prepare", "quantize_layer", "pack", "dequant_gemv", "Workspace",
           "NotPositiveDefinite", "GPTQError"]
