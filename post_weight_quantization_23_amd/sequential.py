"""Layer-by-layer GPTQ over a stack of gated MLP blocks, every step a HIP kernel.

The pages: "What is GPTQ" (queryfeedz glossary), section "How it works" --
layers are quantized in sequence, and the calibration inputs of each one
are what the already-quantized layers before it produce; "Post-Training Quantization:
Calibration, GPTQ and Why Rotations Help", section "Calibration: letting data
pick the rounding" -- one layer at a time keeps memory small.

Block b holds W_gate [h, d], W_up [h, d] and W_down [d, h] and computes
down(silu(gate(x)) * up(x)).  For each block: H of the block input (one SYRK,
shared by gate and up) -> U -> GPTQ of gate and of up -> the quantized gate
and up forwards (the second fused with silu(gate) * up) -> H of that product
-> U -> GPTQ of down -> the quantized down forward, which is the next block's
input.  The forward runs in the activations' 16-bit type: each dequantized
weight matrix is rounded to it once (gptq_round16) and the products read the
16-bit copy (gptq_linear_forward).
This module only sequences calls; the arithmetic is in the library.
"""
from __future__ import annotations

import torch

from . import gptq


def quantize_mlp_stack(X0: torch.Tensor, blocks, bits: int = 4, groupsize: int = 128, percdamp: float = 0.01,
                       act_order: bool = False, blocksize: int = 128, keep: bool = False):
    """X0: calibration tokens [n, d] (bf16/fp16) on the GPU; blocks: list of
    (W_gate, W_up, W_down) device tensors.  Returns (records, X_out): per block
    the gate / up / down quantizer outputs (codes, scales, zeros, g_idx, w_hat)
    and, with keep=True, the block's input X, its Hessian H, the gate output G,
    the product Z and its Hessian H2 (for checking); X_out is the last block's
    quantized output."""
    ws_h, ws_p, ws_q = gptq.Workspace(), gptq.Workspace(), gptq.Workspace()
    X = X0
    records = []
    for Wg, Wu, Wd in blocks:
        d = X.shape[1]
        U = torch.zeros((d, d), dtype=torch.float32, device=X.device)
        gptq.hessian_accumulate(U, X, ws=ws_h)
        H = U.clone() if keep else None
        perm, dead, _ = gptq.prepare(U, percdamp, act_order, ws=ws_p)      # H -> U in place
        qg = gptq.quantize_layer(Wg, U, perm, dead, bits, groupsize, blocksize, want_w_hat=True, ws=ws_q)
        qu = gptq.quantize_layer(Wu, U, perm, dead, bits, groupsize, blocksize, want_w_hat=True, ws=ws_q)
        w16 = gptq.round16(qg["w_hat"], X.dtype)
        G = gptq.linear_forward(X, w16)
        gptq.round16(qu["w_hat"], X.dtype, out=w16)
        Z = gptq.linear_forward(X, w16, gate=G)
        h = Z.shape[1]
        U2 = torch.zeros((h, h), dtype=torch.float32, device=X.device)
        gptq.hessian_accumulate(U2, Z, ws=ws_h)
        H2 = U2.clone() if keep else None
        perm2, dead2, _ = gptq.prepare(U2, percdamp, act_order, ws=ws_p)
        qd = gptq.quantize_layer(Wd, U2, perm2, dead2, bits, groupsize, blocksize, want_w_hat=True, ws=ws_q)
        Xn = gptq.linear_forward(Z, gptq.round16(qd["w_hat"], Z.dtype))
        rec = {"gate": qg, "up": qu, "down": qd, "U": U, "perm": perm, "U2": U2, "perm2": perm2}
        if keep:
            rec.update({"X": X, "H": H, "G": G, "Z": Z, "H2": H2})
        records.append(rec)
        X = Xn
    return records, X
