"""Sign flip + orthonormal Walsh-Hadamard rotation of a 128-element group.

mlxcel PR #369 ("Change", and the commit "use rotated-codec-basis SDPA for
Turbo4Asym decode") stores the codes in a "WHT-rotated basis" and undoes it
with an inverse Walsh-Hadamard transform; the advisor commit (#376) notes the
transform needs a power-of-two head dim.  The sign pattern and the ordering
are not printed.  Readings taken here: natural (Sylvester) ordering,
H_ij = (-1)^popcount(i & j), normalised by 1/sqrt(128); the Rademacher signs
are applied before H on the way in and after H on the way out:

    rotate(x)  = H (s * x) / sqrt(128)
    inverse(y) = s * (H y) / sqrt(128)

H is symmetric and H H = 128 I, so inverse(rotate(x)) = x.
"""
import math

import numpy as np

HEAD_DIM = 128
SQRT_D = math.sqrt(HEAD_DIM)


def sylvester(n: int = HEAD_DIM) -> np.ndarray:
    """Unnormalised Sylvester Hadamard matrix (entries +-1, int64), built by H2n = [[H, H], [H, -H]]."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht(x: np.ndarray) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform along the last axis (butterfly).

    Same dtype in and out; for integer input the result is exact."""
    y = np.array(x, copy=True)
    n = y.shape[-1]
    h = 1
    while h < n:
        y = y.reshape(y.shape[:-1] + (n // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (n,))
        h *= 2
    return y


def rotate_unnormalised(x, signs) -> np.ndarray:
    """H (s * x) in float64.  For fp16 x this is exact: every term is a multiple of
    2**-24 below 2**16, so partial sums of 128 terms need at most 47 bits."""
    h = sylvester().astype(np.float64)
    return (np.asarray(x, dtype=np.float64) * np.asarray(signs, dtype=np.float64)) @ h


def rotate(x, signs) -> np.ndarray:
    """Forward rotation into the codec basis: H (s * x) / sqrt(128), float64."""
    return rotate_unnormalised(x, signs) / SQRT_D


def inverse_rotate(y, signs) -> np.ndarray:
    """Back to the original basis: s * (H y) / sqrt(128), float64."""
    h = sylvester().astype(np.float64)
    return (np.asarray(y, dtype=np.float64) @ h) / SQRT_D * np.asarray(signs, dtype=np.float64)
