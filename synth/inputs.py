"""Seeded synthetic layers and calibration activations.

Shared by the tests, the smoke check and the benchmark: the oracle and the HIP
path are always fed the SAME tensors made here.  This module holds none of the
quantizer's arithmetic -- only random numbers shaped like the workloads the
GPTQ pages describe ("GPTQ, with the code open", sections "Measuring damage
where it matters" and "Paper vs. code": 128 calibration chunks of 2048 tokens;
7B-class and OPT-175B-class linear layers).  No dataset and no trained weights
are used: weights are N(0, 0.02^2), activations are Student-t(4) with a few
loud "outlier" input channels (the heavy-tailed, outlier-ridden activations
the pages talk about), or ReLU-sparse for an MLP down projection.

Seeds: numpy.random.SeedSequence([workload_id, layer, stream]) with stream 0
for W, 1 for X, 2 for the choice of outlier channels.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

T4_Q60 = 0.2707  # 60th percentile of Student-t(4): relu(t - q60) is 60 % zeros


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int            # workload id used in the seed
    rows: int           # outputs (r)
    cols: int           # inputs (c = d)
    tokens: int         # calibration tokens (N)
    w_dtype: str        # "float32" | "bfloat16" | "float16"
    x_dtype: str
    x_kind: str         # "normal" | "t4" | "t4_relu"
    outliers: int       # number of outlier input channels
    outlier_gain: float
    bits: int
    groupsize: int      # <= 0: one ruler per row
    blocksize: int
    percdamp: float
    act_order: bool


WORKLOADS = {
    # single small layer: fp32, 128 x 256, 2048 tokens, 4 loud channels x20
    "tiny_fp32_128x256": Workload("tiny_fp32_128x256", 1, 128, 256, 2048, "float32", "float32",
                                  "normal", 4, 20.0, 4, -1, 128, 0.01, False),
    # Llama-7B-shaped attention projection, 128 x 2048 calibration tokens
    "llama7b_attn_4096x4096": Workload("llama7b_attn_4096x4096", 2, 4096, 4096, 262144, "bfloat16",
                                       "bfloat16", "t4", 20, 30.0, 4, 128, 128, 0.01, False),
    # Llama-7B-shaped MLP pair, 3-bit, act-order
    "llama7b_up_11008x4096": Workload("llama7b_up_11008x4096", 3, 11008, 4096, 262144, "bfloat16",
                                      "bfloat16", "t4", 20, 30.0, 3, 128, 128, 0.01, True),
    "llama7b_down_4096x11008": Workload("llama7b_down_4096x11008", 4, 4096, 11008, 262144, "bfloat16",
                                        "bfloat16", "t4_relu", 0, 1.0, 3, 128, 128, 0.01, True),
    # OPT-175B-shaped layers, fp16, 3-bit
    "opt175b_out_12288x12288": Workload("opt175b_out_12288x12288", 5, 12288, 12288, 262144, "float16",
                                        "float16", "t4", 12, 50.0, 3, 128, 128, 0.01, False),
    "opt175b_fc2_12288x49152": Workload("opt175b_fc2_12288x49152", 6, 12288, 49152, 262144, "float16",
                                        "float16", "t4", 49, 50.0, 3, 128, 128, 0.01, False),
}


def seed_sequence(wid: int, layer: int, stream: int) -> np.random.SeedSequence:
    return np.random.SeedSequence([int(wid), int(layer), int(stream)])


def torch_seed(wid: int, layer: int, stream: int) -> int:
    return int(seed_sequence(wid, layer, stream).generate_state(1, np.uint64)[0] & ((1 << 63) - 1))


def outlier_channels(d: int, count: int, wid: int, layer: int = 0) -> np.ndarray:
    rng = np.random.default_rng(seed_sequence(wid, layer, 2))
    return np.sort(rng.choice(d, size=min(count, d), replace=False))


# --------------------------------------------------------------------------
# Host (NumPy) generation -- small and medium shapes.  Returns float32 arrays
# whose values are already representable in the requested storage dtype
# (bf16/fp16 rounding happens once, with round-half-even, in torch).
# --------------------------------------------------------------------------
def _round_to(arr: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "float32":
        return arr.astype(np.float32)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(getattr(torch, dtype)).to(torch.float32).numpy()


def weights_host(rows: int, cols: int, wid: int = 0, layer: int = 0, dtype: str = "float32",
                 std: float = 0.02) -> np.ndarray:
    rng = np.random.default_rng(seed_sequence(wid, layer, 0))
    return _round_to(rng.standard_normal((rows, cols)) * std, dtype)


def _student_t4(rng, shape):
    z = rng.standard_normal(shape)
    chi = np.zeros(shape)
    for _ in range(4):
        zi = rng.standard_normal(shape)
        chi += zi * zi
    return z / np.sqrt(chi / 4.0)


def activations_host(tokens: int, d: int, kind: str = "normal", outliers: int = 0,
                     gain: float = 1.0, wid: int = 0, layer: int = 0,
                     dtype: str = "float32") -> np.ndarray:
    """Token-major calibration inputs [tokens, d]."""
    rng = np.random.default_rng(seed_sequence(wid, layer, 1))
    if kind == "normal":
        x = rng.standard_normal((tokens, d))
    elif kind == "t4":
        x = _student_t4(rng, (tokens, d))
    elif kind == "t4_relu":
        x = np.maximum(_student_t4(rng, (tokens, d)) - T4_Q60, 0.0)
    else:
        raise ValueError(kind)
    if outliers:
        x[:, outlier_channels(d, outliers, wid, layer)] *= gain
    return _round_to(x, dtype)


def workload_host(w: Workload, layer: int = 0, tokens: int | None = None):
    """(W [rows, cols], X [tokens, cols]) as float32 host arrays."""
    n = w.tokens if tokens is None else tokens
    W = weights_host(w.rows, w.cols, w.wid, layer, w.w_dtype)
    X = activations_host(n, w.cols, w.x_kind, w.outliers, w.outlier_gain, w.wid, layer, w.x_dtype)
    return W, X


# --------------------------------------------------------------------------
# Device (torch) generation -- full-size shapes.  Generated in token chunks so
# the float32 temporaries stay small next to the bf16/fp16 result.
# --------------------------------------------------------------------------
def weights_device(rows: int, cols: int, wid: int, layer: int, dtype: str, device="cuda",
                   std: float = 0.02):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(wid, layer, 0))
    w = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32) * std
    return w.to(getattr(torch, dtype))


def activations_device(tokens: int, d: int, kind: str, outliers: int, gain: float, wid: int,
                       layer: int, dtype: str, device="cuda", chunk_tokens: int = 16384):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(wid, layer, 1))
    out = torch.empty((tokens, d), device=device, dtype=getattr(torch, dtype))
    gainvec = torch.ones(d, device=device, dtype=torch.float32)
    if outliers:
        idx = torch.from_numpy(outlier_channels(d, outliers, wid, layer)).to(device)
        gainvec[idx] = float(gain)
    for s in range(0, tokens, chunk_tokens):
        n = min(chunk_tokens, tokens - s)
        z = torch.randn((n, d), generator=g, device=device, dtype=torch.float32)
        if kind == "normal":
            x = z
        else:
            chi = torch.zeros_like(z)
            for _ in range(4):
                zi = torch.randn((n, d), generator=g, device=device, dtype=torch.float32)
                chi.addcmul_(zi, zi)
            x = z / torch.sqrt(chi * 0.25)
            if kind == "t4_relu":
                x = torch.clamp_min(x - T4_Q60, 0.0)
            elif kind != "t4":
                raise ValueError(kind)
        out[s:s + n] = (x * gainvec).to(out.dtype)
    return out


# The 7B-shaped decoder sweep: 32 blocks x 7 linear layers, 4-bit g128, each
# linear with its own weights and its own calibration activations (seeded by
# its position 7 * block + k), Student-t(4) with 0.5 % outlier channels x30.
LLAMA7B_BLOCK = (("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
                 ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008))


def llama7b_sweep(blocks: int = 32):
    """[(Workload, layer index)] for every linear of the sweep, in model order."""
    out = []
    for b in range(blocks):
        for k, (name, r, c) in enumerate(LLAMA7B_BLOCK):
            w = Workload(f"llama7b_sweep_{name}_{r}x{c}", 7, r, c, 262144, "bfloat16", "bfloat16", "t4",
                         int(round(0.005 * c)), 30.0, 4, 128, 128, 0.01, False)
            out.append((w, 7 * b + k))
    return out


def workload_device(w: Workload, layer: int = 0, tokens: int | None = None, device="cuda"):
    n = w.tokens if tokens is None else tokens
    W = weights_device(w.rows, w.cols, w.wid, layer, w.w_dtype, device)
    X = activations_device(n, w.cols, w.x_kind, w.outliers, w.outlier_gain, w.wid, layer,
                           w.x_dtype, device)
    return W, X


# --------------------------------------------------------------------------
# Packed layers for the dequantizing matrix-vector product (one generated
# token through a quantized linear layer).  Codes are uniform ticks; scales
# are log-normal around the tick width of a 128-weight N(0, 0.02^2) row slice
# (range ~ 5 sigma over 2^b - 1 ticks); zero points are uniform ticks; the
# act-order permutation is uniform.  x is one token of the activation recipe
# above.  Seeds: SeedSequence([seed, 0, 3]) for the layer, ([seed, 0, 4]) for x.
# --------------------------------------------------------------------------
def n_groups(cols: int, groupsize: int) -> int:
    return (cols + groupsize - 1) // groupsize if 0 < groupsize < cols else 1


def packed_layer_host(rows: int, cols: int, bits: int, groupsize: int, seed: int, act_order: bool = False):
    """(codes uint8 [rows, cols], scales fp32 [rows, G], zeros int32 [rows, G], perm int32 [cols] | None)."""
    rng = np.random.default_rng(seed_sequence(seed, 0, 3))
    G = n_groups(cols, groupsize)
    codes = rng.integers(0, 2 ** bits, size=(rows, cols), dtype=np.uint8)
    width = 0.02 * 5.0 / (2 ** bits - 1)
    scales = (width * np.exp(0.3 * rng.standard_normal((rows, G)))).astype(np.float32)
    zeros = rng.integers(0, 2 ** bits, size=(rows, G)).astype(np.int32)
    perm = rng.permutation(cols).astype(np.int32) if act_order else None
    return codes, scales, zeros, perm


def packed_layer_device(rows: int, cols: int, bits: int, groupsize: int, seed: int, act_order: bool = False,
                        device="cuda"):
    """Device twin of packed_layer_host for full-size shapes (torch generator)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(seed, 0, 3))
    G = n_groups(cols, groupsize)
    codes = torch.randint(0, 2 ** bits, (rows, cols), generator=g, device=device, dtype=torch.uint8)
    width = 0.02 * 5.0 / (2 ** bits - 1)
    scales = width * torch.exp(0.3 * torch.randn((rows, G), generator=g, device=device))
    zeros = torch.randint(0, 2 ** bits, (rows, G), generator=g, device=device, dtype=torch.int32)
    perm = torch.randperm(cols, generator=g, device=device).to(torch.int32) if act_order else None
    return codes, scales.float(), zeros, perm


def token_host(cols: int, seed: int, dtype: str, kind: str = "t4", outliers: int = 0, gain: float = 1.0):
    """One activation vector [cols] (float32 values representable in dtype)."""
    rng = np.random.default_rng(seed_sequence(seed, 0, 4))
    x = _student_t4(rng, (cols,)) if kind != "normal" else rng.standard_normal(cols)
    if kind == "t4_relu":
        x = np.maximum(x - T4_Q60, 0.0)
    if outliers:
        x[outlier_channels(cols, outliers, seed, 0)] *= gain
    return _round_to(x, dtype)
