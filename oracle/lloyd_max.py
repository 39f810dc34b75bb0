"""Lloyd-Max scalar quantizer for a Gaussian source, and the frozen codebooks.

The pages describe the codec's dequant as "codebook entry at the index, times
the group norm" with a symmetric 4-magnitude table for the 3-bit format
(turboquant_plus, "SMEM Pre-Dequant Experiment", section "What Would Actually
Work" item 1 and "Also Implemented: Q-Centroid Precompute", which indexes
mag[c] for c = 0..3), and a 16-centroid 4-bit variant (mlxcel PR #369,
"Result").  They print no centroid values.  Reading taken here: the levels
are the Lloyd-Max (minimum-MSE) quantizer of one coordinate of a rotated unit
vector in 128 dimensions, modelled as N(0, 1/128); they are designed for
N(0, 1) in float64, scaled by 1/sqrt(128), then rounded to fp16, and the fp16
values are the codebook both sides use.
"""
import math

import numpy as np
from scipy.special import ndtr

_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)
HEAD_DIM = 128


def _pdf(x):
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    fin = np.isfinite(x)
    out[fin] = np.exp(-0.5 * x[fin] * x[fin]) * _INV_SQRT_2PI
    return out


def _upper_tail(x):
    """P(X > x) for X ~ N(0,1); accurate for large positive x."""
    return ndtr(-np.asarray(x, dtype=np.float64))


def cell_moments(a, b):
    """Zeroth, first and second moments of N(0,1) restricted to [a, b], 0 <= a < b <= inf."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    p = _upper_tail(a) - _upper_tail(b)
    e1 = _pdf(a) - _pdf(b)
    bphi = np.zeros_like(b)
    fin = np.isfinite(b)
    bphi[fin] = b[fin] * _pdf(b[fin])
    e2 = p + a * _pdf(a) - bphi
    return p, e1, e2


def lloyd_max_normal(levels: int, tol: float = 1e-15, max_iter: int = 2_000_000):
    """Lloyd-Max levels for N(0,1): returns (centroids ascending, boundaries, iterations).

    The positive half is solved and mirrored, so the result is exactly
    symmetric.  Iteration (Lloyd's method I): each boundary is the midpoint of
    its two neighbouring centroids; each centroid is the conditional mean of
    its cell.  Starts from equiprobable cells.
    """
    if levels < 2 or levels % 2:
        raise ValueError("levels must be even and >= 2")
    half = levels // 2
    # equiprobable cells on [0, inf): boundaries at the (0.5 + k/(2 half)) quantiles
    from scipy.special import ndtri
    bnd = np.concatenate([[0.0], ndtri(0.5 + 0.5 * np.arange(1, half) / half), [np.inf]])
    c = np.zeros(half)
    it = 0
    for it in range(1, max_iter + 1):
        p, e1, _ = cell_moments(bnd[:-1], bnd[1:])
        c_new = e1 / p
        change = float(np.max(np.abs(c_new - c)))
        c = c_new
        bnd[1:-1] = 0.5 * (c[:-1] + c[1:])
        if change < tol:
            break
    full = np.concatenate([-c[::-1], c])
    inner = np.concatenate([-bnd[1:-1][::-1], [0.0], bnd[1:-1]])
    return full, inner, it


def mse_normal(codebook_ascending) -> float:
    """E[(X - Q(X))^2] for X ~ N(0,1) under nearest-neighbour quantization to the given levels.

    Works for any symmetric ascending codebook (cells are split at midpoints)."""
    c = np.asarray(codebook_ascending, dtype=np.float64)
    if not np.allclose(c, -c[::-1], rtol=0, atol=0):
        raise ValueError("codebook must be symmetric")
    half = len(c) // 2
    pos = c[half:]
    bnd = np.concatenate([[0.0], 0.5 * (pos[:-1] + pos[1:]), [np.inf]])
    p, e1, e2 = cell_moments(bnd[:-1], bnd[1:])
    return float(2.0 * np.sum(e2 - 2.0 * pos * e1 + pos * pos * p))


def frozen_codebook(bits: int) -> np.ndarray:
    """The codebook as both sides use it: fp16 values, ascending, 2**bits entries.

    Lloyd-Max for N(0,1) scaled by 1/sqrt(128) (one coordinate of a rotated
    unit vector), rounded to nearest-even fp16."""
    c, _, _ = lloyd_max_normal(2 ** bits)
    return (c / math.sqrt(HEAD_DIM)).astype(np.float16)


def decision_boundaries(codebook16) -> np.ndarray:
    """Midpoints between adjacent fp16 codebook entries, in float64 (exact)."""
    c = np.asarray(codebook16, dtype=np.float16).astype(np.float64)
    return 0.5 * (c[:-1] + c[1:])
