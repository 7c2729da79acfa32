"""MI355X (gfx950) GPTQ layer quantizer: Hessian SYRK, damped inverse Cholesky
factor, lazy-block quantize-and-repair, int3/int4 packing, the dequantizing
matrix-vector product over the packed words, the Hadamard pre-rotation and the
quantized forward for layer-by-layer calibration, as hand-written HIP kernels
behind the C ABI in include/gptq.h."""
from .gptq import (GPTQError, NotPositiveDefinite, Workspace, dequant_gemv, hadamard_rotate, hessian_accumulate,
                   linear_forward, pack, prepare, prepare_noalloc, quantize_layer, round16)
from .sequential import quantize_mlp_stack

__all__ = ["hessian_accumulate", "prepare", "prepare_noalloc", "quantize_layer", "pack", "dequant_gemv", "hadamard_rotate",
           "linear_forward", "round16", "quantize_mlp_stack", "Workspace",
           "NotPositiveDefinite", "GPTQError"]
