"""Python binding of the gfx950 GPTQ layer quantizer (argument marshalling only).

The names follow the C ABI in include/gptq.h; every step runs in the HIP
library.  Tensors must live on the current HIP device; work is enqueued on
torch's current stream.  Method: the GPTQ layer quantizer of "GPTQ, with the
code open" (sections "Measuring damage where it matters", "The repair rule",
"From one repair to a whole model", "Paper vs. code").
"""
from __future__ import annotations

import ctypes as C

import torch

from . import _lib
from ._lib import GPTQ_BF16, GPTQ_F16, GPTQ_F32, GPTQError

__all__ = ["hessian_accumulate", "prepare", "prepare_noalloc", "quantize_layer", "pack", "dequant_gemv", "hadamard_rotate",
           "linear_forward", "Workspace",
           "NotPositiveDefinite", "GPTQError"]

_DT = {torch.float32: GPTQ_F32, torch.bfloat16: GPTQ_BF16, torch.float16: GPTQ_F16}


class NotPositiveDefinite(RuntimeError):
    """The damped Hessian has no Cholesky factor (info > 0) or holds NaN/Inf (info < 0)."""


def _ptr(t):
    return C.c_void_p(0 if t is None else t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype=None, ndim=None, dev=None, on_gpu=True):
    """Type, dtype and rank of one argument; then (on_gpu) its device."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D")
    if on_gpu:
        _on_gpu(t, name, dev)


def _on_gpu(t, name, dev=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")


class Workspace:
    """A reusable device scratch buffer (grown on demand, 256-byte aligned)."""

    def __init__(self, device=None):
        self.device = device
        self.buf = None

    def get(self, nbytes: int, device):
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        return self.buf, self.buf.numel()


def _ws(ws, nbytes, device):
    if ws is None:
        ws = Workspace()
    return ws.get(nbytes, device)


def hessian_accumulate(H: torch.Tensor, X: torch.Tensor, ws: Workspace | None = None) -> None:
    """H[i][j] += 2 sum_t X[t][i] X[t][j] on the upper triangle (H fp32 [d, d], X [N, d])."""
    _need(H, "H", torch.float32, 2)
    _need(X, "X", None, 2, H.device)
    if X.dtype not in _DT:
        raise TypeError("X must be float32, bfloat16 or float16")
    d = H.shape[0]
    if H.shape != (d, d) or not H.is_contiguous():
        raise ValueError("H must be a contiguous square matrix")
    if X.shape[1] != d or X.stride(1) != 1:
        raise ValueError("X must be [tokens, d] with unit feature stride")
    n = X.shape[0]
    xt = _DT[X.dtype]
    need = _lib.query("gptq_hessian_workspace_size", d, n, xt)
    buf, nb = _ws(ws, need, H.device)
    _lib.call("gptq_hessian_accumulate", _ptr(H), d, _ptr(X), xt, n, X.stride(0), _ptr(buf), nb, _stream())


def prepare(H: torch.Tensor, percdamp: float = 0.01, act_order: bool = False, check: bool = True,
            ws: Workspace | None = None):
    """Replace H (fp32 [d, d], upper triangle) by U = chol_upper(H_damped^{-1}) in place.

    Returns (perm int32 [d], dead uint8 [d], info int32 [1]).  With check=True the
    call synchronises and raises NotPositiveDefinite when info != 0.
    """
    _need(H, "H", torch.float32, 2)
    d = H.shape[0]
    if H.shape != (d, d) or not H.is_contiguous():
        raise ValueError("H must be a contiguous square matrix")
    perm = torch.empty(d, dtype=torch.int32, device=H.device)
    dead = torch.empty(d, dtype=torch.uint8, device=H.device)
    info = torch.empty(1, dtype=torch.int32, device=H.device)
    need = _lib.query("gptq_prepare_workspace_size", d, int(act_order))
    buf, nb = _ws(ws, need, H.device)
    _lib.call("gptq_prepare", _ptr(H), d, float(percdamp), int(act_order), _ptr(perm), _ptr(dead), _ptr(info),
              _ptr(buf), nb, _stream())
    if check:
        v = int(info.item())
        if v != 0:
            raise NotPositiveDefinite(f"gptq_prepare info = {v}")
    return perm, dead, info


def prepare_noalloc(H: torch.Tensor, percdamp: float = 0.01, act_order: bool = False,
                    perm: torch.Tensor | None = None, dead: torch.Tensor | None = None,
                    info: torch.Tensor | None = None):
    """prepare() through the allocation-free entry point (d <= 4096): the
    library's static scratch replaces the workspace.  perm / dead / info may
    be passed preallocated (int32 [d], uint8 [d], int32 [1]); nothing is
    synchronised or checked on the device -- read info afterwards."""
    _need(H, "H", torch.float32, 2, on_gpu=False)
    d = H.shape[0]
    if H.shape != (d, d) or not H.is_contiguous():
        raise ValueError("H must be a contiguous square matrix")
    for t, name, dt, n in ((perm, "perm", torch.int32, d), (dead, "dead", torch.uint8, d),
                           (info, "info", torch.int32, 1)):
        if t is not None:
            _need(t, name, dt, 1, on_gpu=False)
            if t.numel() != n or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous vector of length {n}")
    _on_gpu(H, "H")
    for t, name in ((perm, "perm"), (dead, "dead"), (info, "info")):
        if t is not None:
            _on_gpu(t, name, H.device)
    if perm is None:
        perm = torch.empty(d, dtype=torch.int32, device=H.device)
    if dead is None:
        dead = torch.empty(d, dtype=torch.uint8, device=H.device)
    if info is None:
        info = torch.empty(1, dtype=torch.int32, device=H.device)
    _lib.call("gptq_prepare_noalloc", _ptr(H), d, float(percdamp), int(act_order), _ptr(perm), _ptr(dead),
              _ptr(info), _stream())
    return perm, dead, info


def quantize_layer(W: torch.Tensor, U: torch.Tensor, perm: torch.Tensor | None, dead: torch.Tensor | None,
                   bits: int = 4, groupsize: int = 128, blocksize: int = 128, want_w_hat: bool = False,
                   want_loss: bool = True, ws: Workspace | None = None, out: dict | None = None,
                   sym: bool = False) -> dict:
    """GPTQ-quantize W [r, c] with the factor U from prepare().

    Returns {codes uint8 [r, c], scales fp32 [r, G], zeros int32 [r, G], g_idx int32 [c],
    w_hat fp32 [r, c] or None, row_loss fp32 [r] or None}; outputs are in the
    original column order.  `out` may supply preallocated tensors with those keys.
    `sym` selects the symmetric ruler (zero point at the middle tick).
    """
    # Every shape, dtype and layout is checked before the devices, and all of
    # it before anything is allocated: the kernels index perm, dead and the
    # outputs by r and c, so a short or mis-shaped tensor must not get through.
    _need(W, "W", None, 2, on_gpu=False)
    if W.dtype not in _DT:
        raise TypeError("W must be float32, bfloat16 or float16")
    if W.stride(1) != 1:
        raise ValueError("W must have unit column stride")
    r, c = W.shape
    _need(U, "U", torch.float32, 2, on_gpu=False)
    if U.shape != (c, c) or not U.is_contiguous():
        raise ValueError("U must be a contiguous [c, c] matrix")
    for v, name, dt in ((perm, "perm", torch.int32), (dead, "dead", torch.uint8)):
        if v is not None:
            _need(v, name, dt, 1, on_gpu=False)
            if v.numel() != c or not v.is_contiguous():
                raise ValueError(f"{name} must be a contiguous vector of length c = {c}")
    G = (c + groupsize - 1) // groupsize if groupsize > 0 else 1
    o = dict(out or {})
    unknown = set(o) - {"codes", "scales", "zeros", "g_idx", "w_hat", "row_loss"}
    if unknown:
        raise ValueError(f"unknown output names {sorted(unknown)}")
    shapes = {"codes": ((r, c), torch.uint8), "scales": ((r, G), torch.float32), "zeros": ((r, G), torch.int32),
              "g_idx": ((c,), torch.int32), "w_hat": ((r, c), torch.float32), "row_loss": ((r,), torch.float32)}
    for k, t in o.items():
        if t is None:
            continue
        shape, dt = shapes[k]
        _need(t, f"out[{k!r}]", dt, len(shape), on_gpu=False)
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"out[{k!r}] must be a contiguous {dt} tensor of shape {shape}")
    _on_gpu(W, "W")
    dev = W.device
    for t, name in ((U, "U"), (perm, "perm"), (dead, "dead"), *((t, f"out[{k!r}]") for k, t in o.items())):
        if t is not None:
            _on_gpu(t, name, dev)
    codes = o.get("codes") if o.get("codes") is not None else torch.empty((r, c), dtype=torch.uint8, device=dev)
    scales = o.get("scales") if o.get("scales") is not None else torch.empty((r, G), dtype=torch.float32, device=dev)
    zeros = o.get("zeros") if o.get("zeros") is not None else torch.empty((r, G), dtype=torch.int32, device=dev)
    g_idx = o.get("g_idx") if o.get("g_idx") is not None else torch.empty(c, dtype=torch.int32, device=dev)
    w_hat = o.get("w_hat")
    if want_w_hat and w_hat is None:
        w_hat = torch.empty((r, c), dtype=torch.float32, device=dev)
    row_loss = o.get("row_loss")
    if want_loss and row_loss is None:
        row_loss = torch.empty(r, dtype=torch.float32, device=dev)
    need = _lib.query("gptq_quantize_layer_workspace_size", r, c, blocksize)
    buf, nb = _ws(ws, need, dev)
    _lib.call("gptq_quantize_layer", _ptr(W), _DT[W.dtype], r, c, W.stride(0), _ptr(U), _ptr(perm), _ptr(dead),
              int(bits), int(bool(sym)), int(groupsize), int(blocksize), _ptr(codes), _ptr(scales), _ptr(zeros), _ptr(g_idx),
              _ptr(w_hat), _ptr(row_loss), _ptr(buf), nb, _stream())
    return {"codes": codes, "scales": scales, "zeros": zeros, "g_idx": g_idx, "w_hat": w_hat,
            "row_loss": row_loss}


def pack(codes: torch.Tensor, bits: int, out: torch.Tensor | None = None,
         perm: torch.Tensor | None = None) -> torch.Tensor:
    """Pack uint8 codes [r, c] into uint32 words [r, c*bits/32] (layout in include/gptq.h).

    perm (int32 [c], optional): packed column j takes the code of column
    perm[j] -- pass the act-order permutation to get the layout dequant_gemv
    reads for act-order layers."""
    _need(codes, "codes", torch.uint8, 2)
    if not codes.is_contiguous():
        raise ValueError("codes must be contiguous")
    r, c = codes.shape
    if perm is not None:
        _need(perm, "perm", torch.int32, 1, codes.device)
        if perm.numel() != c or not perm.is_contiguous():
            raise ValueError("perm must be a contiguous int32 vector of length c")
    nw = c * bits // 32
    if out is None:
        out = torch.empty((r, nw), dtype=torch.uint32, device=codes.device)
    _lib.call("gptq_pack", _ptr(codes), r, c, int(bits), _ptr(perm), _ptr(out), out.stride(0), _stream())
    return out


def dequant_gemv(packed: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor, x: torch.Tensor, bits: int,
                 groupsize: int, perm: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """y = W_hat x for a packed layer, dequantizing inside the product (fp32 [r]).

    packed [r, >= c*bits/32] uint32 (pack output), scales fp32 / zeros int32
    [r, n_groups], x bf16 or fp16 [c], perm as given to pack (act-order)."""
    _need(packed, "packed", torch.uint32, 2)
    dev = packed.device
    _need(scales, "scales", torch.float32, 2, dev)
    _need(zeros, "zeros", torch.int32, 2, dev)
    _need(x, "x", None, 1, dev)
    if x.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("x must be bfloat16 or float16")
    if not x.is_contiguous() or packed.stride(1) != 1 or scales.stride(1) != 1 or zeros.stride(1) != 1:
        raise ValueError("x and the rows of packed / scales / zeros must be contiguous")
    if scales.shape != zeros.shape or scales.stride() != zeros.stride():
        raise ValueError("scales and zeros must have the same shape and strides")
    r, c = packed.shape[0], x.numel()
    if scales.shape[0] != r:
        raise ValueError("scales / zeros need one row per packed row")
    if perm is not None:
        _need(perm, "perm", torch.int32, 1, dev)
        if perm.numel() != c or not perm.is_contiguous():
            raise ValueError("perm must be a contiguous int32 vector of length c")
    if out is None:
        out = torch.empty(r, dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, 1, dev)
    if out.numel() != r or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 vector of length r")
    _lib.call("gptq_dequant_gemv", _ptr(packed), r, c, int(bits), packed.stride(0), _ptr(scales), _ptr(zeros),
              scales.stride(0), int(groupsize), _ptr(perm), _ptr(x), _DT[x.dtype], _ptr(out), _stream())
    return out


def hadamard_rotate(A: torch.Tensor, block: int = 0, out: torch.Tensor | None = None,
                    out_dtype: torch.dtype | None = None) -> torch.Tensor:
    """Rows of A [m, d] times blockdiag(H_b / sqrt(b)) (Sylvester H_b); block <= 0
    picks the largest power of two dividing d (at most 8192).  out may be A."""
    _need(A, "A", None, 2)
    if A.dtype not in _DT or A.stride(1) != 1:
        raise ValueError("A must be f32/bf16/f16 with contiguous rows")
    if out is None:
        out = torch.empty(A.shape, dtype=out_dtype or A.dtype, device=A.device)
    _need(out, "out", None, 2, A.device)
    if out.shape != A.shape or out.dtype not in _DT or out.stride(1) != 1:
        raise ValueError("out must match A's shape with contiguous rows")
    m, d = A.shape
    _lib.call("gptq_hadamard_rotate", _ptr(A), _DT[A.dtype], m, d, A.stride(0), int(block), _ptr(out),
              _DT[out.dtype], out.stride(0), _stream())
    return out


def linear_forward(X: torch.Tensor, W_hat: torch.Tensor, gate: torch.Tensor | None = None,
                   out: torch.Tensor | None = None, out_dtype: torch.dtype | None = None) -> torch.Tensor:
    """Y = X W_hat^T over calibration tokens (W_hat rounded to X's 16-bit type,
    fp32 sums), or silu(gate) * round(X W_hat^T) when gate is given.  W_hat is
    fp32, or already rounded to X's type (round16)."""
    _need(X, "X", None, 2)
    dev = X.device
    _need(W_hat, "W_hat", None, 2, dev)
    if X.dtype not in (torch.bfloat16, torch.float16) or X.stride(1) != 1 or W_hat.stride(1) != 1:
        raise ValueError("X must be bf16/fp16 and X, W_hat must have contiguous rows")
    if W_hat.dtype not in (torch.float32, X.dtype):
        raise TypeError("W_hat must be float32 or of X's dtype")
    n, d = X.shape
    r = W_hat.shape[0]
    if W_hat.shape[1] != d:
        raise ValueError("W_hat must be r x d")
    if gate is not None:
        _need(gate, "gate", X.dtype, 2, dev)
        if gate.shape != (n, r) or gate.stride(1) != 1:
            raise ValueError("gate must be n_tok x r with contiguous rows")
    if out is None:
        out = torch.empty((n, r), dtype=out_dtype or X.dtype, device=dev)
    _need(out, "out", None, 2, dev)
    if out.shape != (n, r) or out.dtype not in _DT or out.stride(1) != 1:
        raise ValueError("out must be n_tok x r with contiguous rows")
    _lib.call("gptq_linear_forward", _ptr(X), _DT[X.dtype], n, d, X.stride(0), _ptr(W_hat), _DT[W_hat.dtype], r,
              W_hat.stride(0), 1 if gate is not None else 0, _ptr(gate), gate.stride(0) if gate is not None else 0,
              _ptr(out), _DT[out.dtype], out.stride(0), _stream())
    return out


def round16(src: torch.Tensor, dtype: torch.dtype, out: torch.Tensor | None = None) -> torch.Tensor:
    """src (fp32, 2-D, contiguous rows) rounded to bf16 / fp16, round-to-nearest-even."""
    _need(src, "src", torch.float32, 2)
    if dtype not in (torch.bfloat16, torch.float16) or src.stride(1) != 1:
        raise ValueError("dtype must be bf16 or fp16 and src must have contiguous rows")
    rows, cols = src.shape
    if out is None:
        out = torch.empty((rows, cols), dtype=dtype, device=src.device)
    _need(out, "out", dtype, 2, src.device)
    if out.shape != src.shape or out.stride(1) != 1:
        raise ValueError("out must match src's shape with contiguous rows")
    _lib.call("gptq_round16", _ptr(src), rows, cols, src.stride(0), _DT[dtype], _ptr(out), out.stride(0), _stream())
    return out

