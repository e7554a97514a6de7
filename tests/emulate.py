"""Independent pins for the oracle (no code shared with ``oracle/``).

``fold_f64_emulated`` computes the order contract through binary64: the
product of a binary32 (or bfloat16) a and a bfloat16 w is exact in binary64
(at most 24 + 8 significant bits), rounding it to binary32 gives the product's
single binary32 rounding; the binary64 sum of two binary32 values rounded to
binary32 is the correctly rounded binary32 sum, because binary64 carries
53 >= 2*24 + 2 bits (S. A. Figueroa, "When is double rounding innocuous?",
SIGNUM Newsletter 30(3), 1995). So this loop reproduces the binary32 fold bit
for bit from expressions that share nothing with the C oracle.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def widen(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f64(A: np.ndarray) -> np.ndarray:
    if A.dtype == np.uint16:
        return widen(A).astype(np.float64)
    assert A.dtype == np.float32
    return A.astype(np.float64)


def fold_f64_emulated(A: np.ndarray, W: np.ndarray, reverse: bool = False) -> np.ndarray:
    a = as_f64(A)                   # [M, K]
    w = widen(W).astype(np.float64)  # [K, N]
    M, K = a.shape
    acc = np.zeros((M, w.shape[1]), dtype=np.float32)
    ks = range(K - 1, -1, -1) if reverse else range(K)
    for k in ks:
        p = (a[:, k:k + 1] * w[k:k + 1, :]).astype(np.float32)           # exact, then one rounding
        acc = (acc.astype(np.float64) + p.astype(np.float64)).astype(np.float32)
    return acc


def exact_dot(a_vals, w_vals) -> Fraction:
    return sum((Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a_vals, w_vals)), Fraction(0))


def bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
