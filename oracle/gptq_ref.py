"""CPU oracle of the GPTQ layer quantizer.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The product path (the HIP library and its Python binding) never
imports, calls or links it, and this module imports nothing from the product
package.  It is deliberately plain and slow: NumPy, float64, one column at a
time, no blocking beyond what the method itself states.

Sources (the pages are cited by title and section):

* "GPTQ, with the code open" (modelfoundations.com/notes/gptq) -- the only page
  that describes the method at the level of formulas and loop structure:
  - section "What quantization is, and why anyone bothers": the min-max ruler,
    the zero point rounded to a whole tick, dequantisation scale*(q - zero);
  - section "The obvious approach, and how it fails": round-to-nearest;
  - section "Measuring damage where it matters": H = 2 X X^T prices the output
    damage of weight errors and is shared by every row;
  - section "The repair rule": the Optimal-Brain-Surgeon adjustment of the
    still-free weights after one weight is forced onto a tick;
  - section "From one repair to a whole model": one fixed left-to-right column
    order for all rows, the Cholesky factor of the inverse holding every
    number the shrinking inverses need, the per-weight loss (w-q)^2/(2 d^2),
    immediate repairs inside a block of 128 columns with the rest deferred
    to one matrix product, and rulers fitted before any repair;
  - section "Paper vs. code": dead inputs zeroed, 1 % damping of the mean
    diagonal, full fp32 arithmetic (no TF32), asymmetric min-max rulers whose
    range always includes 0, act-order, and rulers per group of columns.
* "What is GPTQ" (queryfeedz glossary), table "Key settings": bits 3/4/8,
  group size 128/64/32, act-order.
* apxml course chapter "intro-gptq": the layer objective ||W X - W_q X||^2.

Readings where the pages are silent:

* H is the raw 2 * sum_t x_t x_t^T, never rescaled to a running mean (the
  pages call the two the same matrix up to a harmless constant factor).
* A dead input is one whose H diagonal is exactly 0; its diagonal is set to 1
  before damping, its weights to 0.  A per-row ruler is fitted on the
  original weights, before that zeroing.
* Act-order is a stable descending sort of diag(H) (ties: lower index first),
  taken after the dead-input fix and before damping.  Groups are runs of
  `groupsize` columns in processing (permuted) order.
* A group's ruler is fitted when the column loop reaches the group's first
  column, on the current (already repaired) values of its columns.
* Ties round half to even, for the code and for the zero point; the code is
  rne(w/scale) + zero, then clamped to [0, 2^b - 1].  An all-zero range uses
  [-1, 1].
* The symmetric ruler (an option the page names without a formula) uses the
  range [-m, m], m = max|w|, and the middle tick 2^(b-1) as its zero point.
* Precision of decisions: the page's code runs in full fp32, so every step that
  turns floating point into an integer -- the ruler (min, max, scale, zero)
  and the division w/scale that picks a tick -- is evaluated in IEEE fp32 here
  too.  Everything continuous (H, the inverse factor, the repairs, the losses)
  is float64.
"""
from __future__ import annotations

import itertools

import numpy as np

F32 = np.float32
F64 = np.float64

__all__ = [
    "NotPositiveDefinite",
    "hessian",
    "fit_ruler",
    "round_to_grid",
    "dequantize",
    "prepare",
    "upper_cholesky_of_inverse",
    "gptq_quantize",
    "TieReplay",
    "rtn",
    "layer_loss",
    "layer_loss_from_x",
    "obs_repair",
    "lstsq_repair",
    "brute_force_row",
    "pack_codes",
    "unpack_codes",
    "dequant_gemv",
    "hadamard",
    "default_hadamard_block",
    "hadamard_rotate",
    "round16",
    "silu",
    "linear_forward",
    "quantize_mlp_stack",
]


class NotPositiveDefinite(ValueError):
    """The damped Hessian (or its inverse) has no Cholesky factor."""


# ---------------------------------------------------------------------------
# Hessian -- "Measuring damage where it matters": H = 2 X X^T, X holding the
# calibration inputs.  Memory layout here is token-major [N, d] (one row per
# token), so X X^T of the page is sum over tokens of x_t x_t^T.
# ---------------------------------------------------------------------------
def hessian(X, chunk: int = 1 << 15) -> np.ndarray:
    """Return H = 2 * sum_t x_t x_t^T (float64, full symmetric d x d).

    X is token-major [N, d] in any real dtype; values are promoted exactly.
    """
    X = np.asarray(X)
    if X.ndim != 2:
        raise ValueError("X must be 2-D [tokens, features]")
    n, d = X.shape
    acc = np.zeros((d, d), F64)
    for s in range(0, n, chunk):
        x = X[s:s + chunk].astype(F64)
        acc += x.T @ x
    return 2.0 * acc


# ---------------------------------------------------------------------------
# The ruler -- "What quantization is, and why anyone bothers" and the
# "Paper vs. code" notes: 2^b evenly spaced ticks over [min, max] of the row
# (or group), the range stretched to include 0, the zero point rounded to a
# whole tick, w_hat = scale * (q - zero).
# ---------------------------------------------------------------------------
def fit_ruler(w, bits: int, sym: bool = False):
    """Fit one min-max ruler per row of `w` ([rows, k], k >= 1).

    Asymmetric (the default): the range [min, max] stretched to include 0,
    scale = (max - min) / (2^b - 1), zero = rne(-min / scale).
    Symmetric (the pages name the option without a formula; plainest reading):
    the range [-m, m] with m = max(|min|, |max|), scale = 2m / (2^b - 1), and
    the zero point the middle tick 2^(b-1), so 0.0 stays exactly on a tick.
    An all-zero range uses [-1, 1] in both modes.

    Returns (scale fp32 [rows], zero float [rows] holding whole numbers,
    zero_unrounded fp32 [rows]).  Evaluated in fp32 (see module docstring).
    """
    w32 = np.asarray(w, dtype=F64).astype(F32)
    if w32.ndim != 2 or w32.shape[1] == 0:
        raise ValueError("fit_ruler needs a non-empty [rows, k] array")
    xmin = np.minimum(w32.min(axis=1), F32(0.0))
    xmax = np.maximum(w32.max(axis=1), F32(0.0))
    if sym:
        m = np.maximum(-xmin, xmax).astype(F32)
        xmin, xmax = (-m).astype(F32), m
    flat = (xmin == 0) & (xmax == 0)
    xmin = np.where(flat, F32(-1.0), xmin).astype(F32)
    xmax = np.where(flat, F32(1.0), xmax).astype(F32)
    maxq = F32(2 ** bits - 1)
    scale = ((xmax - xmin) / maxq).astype(F32)
    if sym:
        zero_t = np.full(scale.shape, F32(2 ** (bits - 1)), F32)
    else:
        zero_t = (-xmin / scale).astype(F32)
    zero = np.rint(zero_t).astype(F64)
    return scale, zero, zero_t


def round_to_grid(w, scale, zero, bits: int):
    """Nearest tick: q = clamp(rne(w / scale) + zero, 0, 2^b - 1).

    The division is fp32 (see module docstring).  Returns (q float64 holding
    whole numbers, t = w/scale in fp32).
    """
    t = (np.asarray(w, dtype=F64).astype(F32) / np.asarray(scale, F32)).astype(F32)
    q = np.clip(np.rint(t).astype(F64) + zero, 0, 2 ** bits - 1)
    return q, t


def dequantize(q, scale, zero):
    """w_hat = scale * (q - zero), in float64 from the fp32 scale."""
    return np.asarray(scale, F32).astype(F64) * (np.asarray(q, F64) - zero)


# ---------------------------------------------------------------------------
# Preparation of H -- "Paper vs. code": dead inputs, act-order, damping;
# "From one repair to a whole model": the Cholesky factor of the inverse.
# ---------------------------------------------------------------------------
def upper_cholesky_of_inverse(Hd) -> np.ndarray:
    """U upper triangular with U^T U = Hd^{-1}.

    Follows the page's three steps literally: Cholesky of Hd, inverse from
    that factor, Cholesky of the inverse taken in its upper form.
    """
    Hd = np.asarray(Hd, F64)
    try:
        L = np.linalg.cholesky(Hd)
    except np.linalg.LinAlgError as exc:
        raise NotPositiveDefinite("damped H is not positive definite") from exc
    Linv = np.linalg.inv(L)                     # lower triangular
    Hinv = Linv.T @ Linv                        # (L L^T)^{-1}
    Hinv = 0.5 * (Hinv + Hinv.T)
    try:
        L2 = np.linalg.cholesky(Hinv)           # Hinv = L2 L2^T
    except np.linalg.LinAlgError as exc:
        raise NotPositiveDefinite("inverse of damped H is not positive definite") from exc
    return np.triu(L2.T)                        # U = L2^T, U^T U = Hinv


def prepare(H_raw, percdamp: float = 0.01, act_order: bool = False):
    """Dead inputs, act-order permutation and damping of H.

    Returns (H_damped in processing order, perm int64[d], dead bool[d],
    damp lambda).  perm[k] is the original column processed k-th.
    """
    H = np.array(H_raw, dtype=F64, copy=True)
    d = H.shape[0]
    dead = np.diag(H) == 0.0
    idx = np.flatnonzero(dead)
    H[idx, idx] = 1.0
    if act_order:
        perm = np.argsort(-np.diag(H), kind="stable")
    else:
        perm = np.arange(d)
    H = H[np.ix_(perm, perm)]
    lam = percdamp * float(np.mean(np.diag(H))) if d else 0.0
    H[np.arange(d), np.arange(d)] += lam
    return H, perm, dead, lam


class TieReplay:
    """Adjudicates codes where two neighbouring ticks are equally valid.

    GPTQ's rounding depends on every earlier repair, so two correct fp32
    implementations can land on different ticks when a value sits at a tick
    midpoint, and every later column of that row then differs.  Given another
    implementation's codes (processing order) and zero points, the oracle
    adopts that choice wherever its own pre-rounding value lies within `band`
    of a midpoint and the other choice is one of the two neighbours; any other
    disagreement is counted as a hard mismatch (the oracle keeps its own).
    """

    def __init__(self, codes_proc, zeros=None, band: float = 1e-3):
        self.codes = np.asarray(codes_proc)
        self.zeros = None if zeros is None else np.asarray(zeros)
        self.band = band
        self.near_ties = 0
        self.hard = 0
        self.zero_near_ties = 0
        self.zero_hard = 0

    def _adjudicate(self, mine, theirs, t, offset, lo, hi):
        diff = mine != theirs
        if not diff.any():
            return mine, 0, 0
        fl = np.floor(t.astype(F64))
        frac = t.astype(F64) - fl
        near = np.abs(frac - 0.5) <= self.band
        lo_n = np.clip(fl + offset, lo, hi)
        hi_n = np.clip(fl + 1.0 + offset, lo, hi)
        ok = diff & near & ((theirs == lo_n) | (theirs == hi_n))
        out = np.where(ok, theirs, mine)
        return out, int(ok.sum()), int((diff & ~ok).sum())

    def code(self, rows, j, q, t, zero, maxq):
        other = self.codes[rows, j].astype(F64)
        q, n_near, n_hard = self._adjudicate(q, other, t, zero, 0.0, float(maxq))
        self.near_ties += n_near
        self.hard += n_hard
        return q

    def zero(self, rows, gidx, zero, zero_t):
        if self.zeros is None:
            return zero
        other = self.zeros[rows, gidx].astype(F64)
        z, n_near, n_hard = self._adjudicate(zero, other, zero_t, 0.0, -np.inf, np.inf)
        self.zero_near_ties += n_near
        self.zero_hard += n_hard
        return z


def gptq_quantize(W0, H_raw, bits: int, groupsize: int = -1, percdamp: float = 0.01,
                  act_order: bool = False, blocksize: int | None = None,
                  U=None, replay: TieReplay | None = None, rows=None, sym: bool = False):
    """Quantize one linear layer with GPTQ.

    W0 [r, c] holds one output per row and one input per column.  H_raw is the
    raw 2 X X^T ([c, c]).  blocksize None runs the plain column-by-column
    method (each repair applied at once to every later column); an integer
    runs the lazy-batch variant (repairs inside the current block at once,
    the rest deferred to one matrix product per block).  U, if given, is the
    upper factor to use (processing order) instead of computing one -- the
    dead-input set and the permutation are still derived from H_raw.
    `rows` (indices into the full layer) is only used to index `replay`.
    `sym` selects the symmetric ruler (see fit_ruler).

    Returns a dict: codes [r, c] (original column order), scales and zeros
    [r, n_groups] (group order = processing order), g_idx [c], w_hat [r, c],
    row_loss [r], perm, dead, lam, U, codes_proc (processing order) and
    pre_round (processing order: each weight's value when its turn came).
    """
    W0 = np.array(W0, dtype=F64, copy=True)
    r, c = W0.shape
    maxq = 2 ** bits - 1
    if rows is None:
        rows = np.arange(r)

    # Per-row ruler, fitted on the original weights before anything else.
    if groupsize <= 0:
        row_scale, row_zero, row_zt = fit_ruler(W0, bits, sym) if c else (None, None, None)
        if replay is not None and c:
            row_zero = replay.zero(rows, 0, row_zero, row_zt)

    Hd, perm, dead, lam = prepare(H_raw, percdamp, act_order)
    W = W0.copy()
    W[:, dead] = 0.0
    W = W[:, perm]
    if U is None:
        U = upper_cholesky_of_inverse(Hd)
    else:
        U = np.asarray(U, F64)

    n_groups = (c + groupsize - 1) // groupsize if groupsize > 0 else 1
    scales = np.zeros((r, n_groups), F32)
    zeros = np.zeros((r, n_groups), F64)
    if groupsize <= 0 and c:
        scales[:, 0] = row_scale
        zeros[:, 0] = row_zero
    Q = np.zeros((r, c), F64)
    What = np.zeros((r, c), F64)
    pre = np.zeros((r, c), F64)
    loss = np.zeros(r, F64)
    scale = row_scale if groupsize <= 0 else None
    zero = row_zero if groupsize <= 0 else None

    B = c if blocksize is None else int(blocksize)
    for i1 in range(0, c, max(B, 1)):
        i2 = min(i1 + B, c) if blocksize is not None else c
        Err = np.zeros((r, i2 - i1), F64)
        for j in range(i1, i2):
            if groupsize > 0 and j % groupsize == 0:
                g = j // groupsize
                scale, zero, zt = fit_ruler(W[:, j:j + groupsize], bits, sym)
                if replay is not None:
                    zero = replay.zero(rows, g, zero, zt)
                scales[:, g] = scale
                zeros[:, g] = zero
            w = W[:, j].copy()
            pre[:, j] = w
            q, t = round_to_grid(w, scale, zero, bits)
            if replay is not None:
                q = replay.code(rows, j, q, t, zero, maxq)
            wq = dequantize(q, scale, zero)
            d_jj = U[j, j]
            loss += (w - wq) ** 2 / (2.0 * d_jj * d_jj)
            e = (w - wq) / d_jj
            # Optimal-Brain-Surgeon repair of every still-free column of this
            # block (all later columns when not lazy).
            W[:, j + 1:i2] -= np.outer(e, U[j, j + 1:i2])
            Err[:, j - i1] = e
            Q[:, j] = q
            What[:, j] = wq
        if blocksize is not None and i2 < c:
            W[:, i2:] -= Err @ U[i1:i2, i2:]

    codes = np.zeros((r, c), np.int64)
    w_hat = np.zeros((r, c), F64)
    codes[:, perm] = Q.astype(np.int64)
    w_hat[:, perm] = What
    g_idx = np.zeros(c, np.int64)
    if groupsize > 0:
        g_idx[perm] = np.arange(c) // groupsize
    return {
        "codes": codes, "scales": scales, "zeros": zeros.astype(np.int64),
        "g_idx": g_idx, "w_hat": w_hat, "row_loss": loss,
        "perm": perm, "dead": dead, "lam": lam, "U": U,
        "codes_proc": Q.astype(np.int64), "pre_round": pre,
    }


# ---------------------------------------------------------------------------
# Round-to-nearest -- "The obvious approach, and how it fails": every weight
# snapped to its nearest tick independently, no repair.  Written separately
# from gptq_quantize on purpose (it pins it).
# ---------------------------------------------------------------------------
def rtn(W, bits: int, groupsize: int = -1, sym: bool = False):
    """Plain round-to-nearest on per-row (groupsize <= 0) or per-group rulers.

    Returns (codes int64 [r, c], w_hat float64 [r, c]).
    """
    W = np.asarray(W, F64)
    r, c = W.shape
    codes = np.zeros((r, c), np.int64)
    w_hat = np.zeros((r, c), F64)
    spans = [(0, c)] if groupsize <= 0 else [(s, min(s + groupsize, c)) for s in range(0, c, groupsize)]
    for a, b in spans:
        scale, zero, _ = fit_ruler(W[:, a:b], bits, sym)
        for j in range(a, b):
            q, _ = round_to_grid(W[:, j], scale, zero, bits)
            codes[:, j] = q.astype(np.int64)
            w_hat[:, j] = dequantize(q, scale, zero)
    return codes, w_hat


# ---------------------------------------------------------------------------
# The layer objective -- apxml "intro-gptq": ||W X - W_q X||^2 (squared
# Frobenius norm over outputs and tokens).
# ---------------------------------------------------------------------------
def layer_loss(W0, W_hat, H_raw) -> float:
    """||(W0 - W_hat) X||_F^2 written through H = 2 X X^T: sum of d^T H d / 2."""
    D = np.asarray(W0, F64) - np.asarray(W_hat, F64)
    return float(0.5 * np.einsum("ri,ij,rj->", D, np.asarray(H_raw, F64), D))


def layer_loss_from_x(W0, W_hat, X) -> float:
    """||(W0 - W_hat) X||_F^2 directly from token-major X [N, d]."""
    D = np.asarray(W0, F64) - np.asarray(W_hat, F64)
    Y = np.asarray(X, F64) @ D.T
    return float(np.sum(Y * Y))


# ---------------------------------------------------------------------------
# Single-repair helpers -- "The repair rule".
# ---------------------------------------------------------------------------
def obs_repair(w, H, q: int, value: float) -> np.ndarray:
    """Force weight q to `value` and move all weights by the OBS rule.

    delta = -(w_q - value) / [H^{-1}]_qq * H^{-1}[:, q]   (all weights free).
    """
    w = np.asarray(w, F64)
    Hinv = np.linalg.inv(np.asarray(H, F64))
    e = w[q] - value
    return w - (e / Hinv[q, q]) * Hinv[:, q]


def lstsq_repair(w, X, q: int, value: float) -> np.ndarray:
    """Same problem as obs_repair, solved by exact least squares.

    Minimise ||X (w' - w)||^2 over w' with w'_q = value; X token-major [N, d].
    """
    w = np.asarray(w, F64)
    X = np.asarray(X, F64)
    e = w[q] - value
    free = [k for k in range(w.size) if k != q]
    # X (w' - w) = X_F delta_F + X_q * (-e) ; choose delta_F to cancel.
    sol, *_ = np.linalg.lstsq(X[:, free], e * X[:, q], rcond=None)
    out = w.copy()
    out[q] = value
    out[free] += sol
    return out


def brute_force_row(w0, X, scale, zero, bits: int):
    """Best code vector for one row on a fixed ruler, by exhaustive search.

    Minimises ||(w0 - w_hat) X||^2 over every code vector (2^b)^d; meant for
    d <= 6.  Returns (codes int64 [d], objective).
    """
    w0 = np.asarray(w0, F64)
    X = np.asarray(X, F64)
    d = w0.size
    levels = np.arange(2 ** bits, dtype=F64)
    grid = np.array(list(itertools.product(levels, repeat=d)), F64)   # [K, d]
    wh = dequantize(grid, scale, zero)
    Y = (w0[None, :] - wh) @ X.T                                       # [K, N]
    obj = np.sum(Y * Y, axis=1)
    k = int(np.argmin(obj))
    return grid[k].astype(np.int64), float(obj[k])


# ---------------------------------------------------------------------------
# Packed storage.  The pages only say that a tick index is stored per weight
# (plus one ruler per row or group); the word layout is this project's:
# little-endian along the input axis, one output row at a time.
#   4 bits: 8 codes per 32-bit word, code k of a word at bits 4k..4k+3.
#   3 bits: 32 codes per three words, code k at bits 3k..3k+2 of the
#           little-endian 96-bit value (word 0 holds bits 0..31).
# Pure-Python integer loops: for small arrays only.
# ---------------------------------------------------------------------------
def pack_codes(codes, bits: int) -> np.ndarray:
    codes = np.asarray(codes)
    r, c = codes.shape
    if bits == 4:
        if c % 8:
            raise ValueError("4-bit packing needs c % 8 == 0")
        out = np.zeros((r, c // 8), np.uint32)
        for i in range(r):
            for wd in range(c // 8):
                v = 0
                for k in range(8):
                    v |= (int(codes[i, 8 * wd + k]) & 0xF) << (4 * k)
                out[i, wd] = v
        return out
    if bits == 3:
        if c % 32:
            raise ValueError("3-bit packing needs c % 32 == 0")
        out = np.zeros((r, 3 * (c // 32)), np.uint32)
        for i in range(r):
            for grp in range(c // 32):
                v = 0
                for k in range(32):
                    v |= (int(codes[i, 32 * grp + k]) & 0x7) << (3 * k)
                for m in range(3):
                    out[i, 3 * grp + m] = (v >> (32 * m)) & 0xFFFFFFFF
        return out
    raise ValueError("packing supports 3 and 4 bits")


def unpack_codes(words, bits: int, c: int) -> np.ndarray:
    words = np.asarray(words)
    r = words.shape[0]
    out = np.zeros((r, c), np.int64)
    if bits == 4:
        for i in range(r):
            for j in range(c):
                out[i, j] = (int(words[i, j // 8]) >> (4 * (j % 8))) & 0xF
        return out
    if bits == 3:
        for i in range(r):
            for grp in range(c // 32):
                v = 0
                for m in range(3):
                    v |= int(words[i, 3 * grp + m]) << (32 * m)
                for k in range(32):
                    out[i, 32 * grp + k] = (v >> (3 * k)) & 0x7
        return out
    raise ValueError("packing supports 3 and 4 bits")


# ---------------------------------------------------------------------------
# Using the packed layer -- "GPTQ, with the code open", section "What
# quantization is, and why anyone bothers": at generation time each weight is
# turned back into scale * (tick - zero) while the matrix-vector product runs
# (a batch-1 product is limited by reading the weights, so reading fewer bits
# is the point).  One ruler per row or per group of input columns; g_idx maps
# each original input column to its group.
# ---------------------------------------------------------------------------
def dequant_gemv(words, bits: int, c: int, scales, zeros, g_idx, x) -> np.ndarray:
    """y = W_hat x in float64 for a packed layer.

    words: packed codes [r, c * bits / 32] (this project's layout, see
    pack_codes); scales/zeros [r, n_groups]; g_idx int [c] (group of each
    input column; all 0 for one ruler per row); x [c].
    """
    codes = unpack_codes(words, bits, c)
    g = np.asarray(g_idx, np.int64)
    w_hat = dequantize(codes, np.asarray(scales)[:, g], np.asarray(zeros, F64)[:, g])
    return w_hat @ np.asarray(x, F64)


# ---------------------------------------------------------------------------
# Hadamard pre-rotation -- "Post-Training Quantization: Calibration, GPTQ and
# Why Rotations Help", sections "Rotations: making outliers disappear" and
# "Why do Hadamard rotations help quantization?": a Hadamard matrix (entries
# +-1, mutually perpendicular rows), scaled to a rotation Q, spreads a lone
# large activation over all entries; rotating the layer's inputs by Q and its
# weights by Q^{-1} = Q^T leaves the product unchanged: (W Q^T)(Q x) = W x.
# Readings: the Sylvester construction (H_1 = [1], H_2k = [[H, H], [H, -H]]),
# Q = H / sqrt(b); a width d that is not a power of two is rotated block-wise,
# Q = blockdiag(H_b / sqrt(b)) with b the largest power of two dividing d.
# Rows of X (token-major) and of W (one row per output) are both rotated along
# their last axis: x_t -> Q x_t and w_i -> Q w_i (Q is symmetric).
# ---------------------------------------------------------------------------
def hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two), entries +-1."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    H = np.ones((1, 1))
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def default_hadamard_block(d: int) -> int:
    """Largest power of two dividing d."""
    return d & -d


def hadamard_rotate(A, block: int | None = None) -> np.ndarray:
    """Each row of A [m, d] times blockdiag(H_b / sqrt(b)), in float64."""
    A = np.asarray(A, F64)
    m, d = A.shape
    b = default_hadamard_block(d) if not block else int(block)
    if d % b:
        raise ValueError("block must divide d")
    Q = hadamard(b) / np.sqrt(b)
    return (A.reshape(m, d // b, b) @ Q.T).reshape(m, d)


# ---------------------------------------------------------------------------
# Layer by layer -- "What is GPTQ" (queryfeedz glossary), section "How it
# works": layers are quantized in sequence, each calibrated on what the
# already-quantized layers before it produce; "Post-Training
# Quantization: Calibration, GPTQ and Why Rotations Help", section
# "Calibration: letting data pick the rounding": the layer's calibration
# inputs are what the (already quantized) model feeds it.
# Readings: the forward pass runs in the model's 16-bit type -- the
# dequantized weights and every layer output are rounded once to it
# (round-to-nearest-even); a gated MLP block is down(silu(gate(x)) * up(x));
# linears that read the same input (gate and up) share one Hessian.
# ---------------------------------------------------------------------------
_MANT = {"bfloat16": 7, "float16": 10, "float32": 23}
_EMIN = {"bfloat16": -126, "float16": -14, "float32": -126}
_MAX = {"bfloat16": (2 - 2.0 ** -7) * 2.0 ** 127, "float16": 65504.0, "float32": float(np.finfo(np.float32).max)}


def round16(x, dtype: str) -> np.ndarray:
    """Round float64 values to the nearest value of `dtype` (ties to even),
    in one step: q = rint(x / ulp) * ulp with ulp the spacing at |x|."""
    x = np.asarray(x, F64)
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    ulp = np.exp2(np.maximum(e, _EMIN[dtype]) - _MANT[dtype])
    y = np.rint(x / ulp) * ulp
    big = np.abs(y) > _MAX[dtype]
    return np.where(big, np.copysign(np.inf, y), y)


def silu(g):
    g = np.asarray(g, F64)
    return g / (1.0 + np.exp(-g))


def linear_forward(X, W_hat, dtype: str, gate=None, out_dtype: str | None = None) -> np.ndarray:
    """X W_hat^T with W_hat rounded once to the 16-bit `dtype`, float64 sums;
    with `gate`: silu(gate) * round(X W_hat^T).  Rounded to out_dtype if given."""
    Wr = round16(W_hat, dtype)
    acc = np.asarray(X, F64) @ Wr.T
    y = acc if gate is None else silu(gate) * round16(acc, dtype)
    return round16(y, out_dtype) if out_dtype else y


def quantize_mlp_stack(X0, blocks, bits: int, groupsize: int = -1, percdamp: float = 0.01,
                       act_order: bool = False, dtype: str = "bfloat16"):
    """GPTQ over a stack of gated MLP blocks (W_gate [h, d], W_up [h, d],
    W_down [d, h]), one layer at a time, each calibrated on the quantized
    outputs of the layers before it.  Returns (records, final output)."""
    X = np.asarray(X0, F64)
    records = []
    for Wg, Wu, Wd in blocks:
        H = hessian(X)                                          # shared by gate and up
        qg = gptq_quantize(Wg, H, bits, groupsize, percdamp, act_order)
        qu = gptq_quantize(Wu, H, bits, groupsize, percdamp, act_order)
        G = linear_forward(X, qg["w_hat"], dtype, out_dtype=dtype)
        Z = linear_forward(X, qu["w_hat"], dtype, gate=G, out_dtype=dtype)
        H2 = hessian(Z)
        qd = gptq_quantize(Wd, H2, bits, groupsize, percdamp, act_order)
        Xn = linear_forward(Z, qd["w_hat"], dtype, out_dtype=dtype)
        records.append({"X": X, "H": H, "gate": qg, "up": qu, "G": G, "Z": Z, "H2": H2, "down": qd})
        X = Xn
    return records, X

