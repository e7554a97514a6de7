"""Python access to the CPU oracle (plain C, see ``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg. The library never imports it.

Arrays are numpy: bfloat16 operands are ``uint16`` bit patterns, binary32 is
``float32``. ``threads > 1`` splits the rows of A over threads; each call of
the C routine covers whole rows, and rows are independent, so the result is
the same bytes as one single-threaded call.
"""
from __future__ import annotations

import ctypes as ct
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import build as _build

_lib = None


def load(path: str | None = None):
    """Load (building if needed) the oracle library; a path loads a specific build."""
    global _lib
    if path is not None:
        return _bind(ct.CDLL(path))
    if _lib is None:
        if not os.path.exists(_build.LIB) or os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC):
            _build.build()
        _lib = _bind(ct.CDLL(_build.LIB))
    return _lib


def _bind(lib):
    P, I64, I = ct.c_void_p, ct.c_int64, ct.c_int
    lib.oracle_source_sha256.restype = ct.c_char_p
    lib.oracle_gemm_ordered.argtypes = [P, I, I64, P, I64, P, I64, I64, I64, I64]
    lib.oracle_gemm_f64.argtypes = [P, I, I64, P, I64, P, I64, I64, I64, I64]
    lib.oracle_gemm_absdot_f64.argtypes = [P, I, I64, P, I64, P, I64, I64, I64, I64]
    lib.oracle_gemv_tree.argtypes = [P, I64, P, I64, P, I64, I64, I64, I64]
    lib.oracle_gemm_mfma.argtypes = [P, I64, P, I64, P, I64, I64, I64, I64]
    lib.oracle_epilogue.argtypes = [P, I64, I64, I64, P, I, P, I64, I, P, I64]
    lib.oracle_ep_exp.argtypes = [ct.c_float]
    lib.oracle_ep_exp.restype = ct.c_float
    lib.oracle_freivalds_prepare.argtypes = [P, I64, I64, I64, P, P, P, P]
    lib.oracle_freivalds_check.argtypes = [P, P, P, P, I64, I64, P, P, ct.c_double, P]
    lib.oracle_freivalds_check.restype = I
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _a_dtype(A: np.ndarray) -> int:
    if A.dtype == np.uint16:
        return 0
    if A.dtype == np.float32:
        return 1
    raise TypeError(f"A must be bf16 bits (uint16) or float32, got {A.dtype}")


def _rows(fn, A, W, out, threads):
    M, K = A.shape
    N = W.shape[1]
    ad = _a_dtype(A)

    def run(r0, r1):
        if r1 > r0:
            fn(_ptr(A[r0:]), ad, max(A.strides[0] // A.itemsize, K), _ptr(W), max(W.strides[0] // W.itemsize, N),
               _ptr(out[r0:]), out.strides[0] // out.itemsize, r1 - r0, N, K)

    if threads <= 1 or M < 2:
        run(0, M)
    else:
        step = (M + threads - 1) // threads
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda r0: run(r0, min(M, r0 + step)), range(0, M, step)))
    return out


def _check(A, W):
    assert A.ndim == 2 and W.ndim == 2 and A.shape[1] == W.shape[0], (A.shape, W.shape)
    assert W.dtype == np.uint16, W.dtype
    # rows may be strided; the inner (k or n) axis must be unit stride
    if A.shape[1] > 1 and A.strides[1] != A.itemsize or A.strides[0] < 0:
        A = np.ascontiguousarray(A)
    if W.shape[1] > 1 and W.strides[1] != W.itemsize or W.strides[0] < 0 or W.shape[1] == 1:
        W = np.ascontiguousarray(W)
    return A, W


def gemm_ordered(A: np.ndarray, W: np.ndarray, threads: int = 1, lib=None) -> np.ndarray:
    """The order-contract product: float32 [M, N]."""
    A, W = _check(A, W)
    out = np.empty((A.shape[0], W.shape[1]), dtype=np.float32)
    return _rows((lib or load()).oracle_gemm_ordered, A, W, out, threads)


def gemm_f64(A: np.ndarray, W: np.ndarray, threads: int = 1) -> np.ndarray:
    A, W = _check(A, W)
    out = np.empty((A.shape[0], W.shape[1]), dtype=np.float64)
    return _rows(load().oracle_gemm_f64, A, W, out, threads)


def gemm_absdot_f64(A: np.ndarray, W: np.ndarray, threads: int = 1) -> np.ndarray:
    A, W = _check(A, W)
    out = np.empty((A.shape[0], W.shape[1]), dtype=np.float64)
    return _rows(load().oracle_gemm_absdot_f64, A, W, out, threads)


ACTS = {"none": 0, "relu": 1, "silu": 2, "gelu_tanh": 3}


def epilogue(Y: np.ndarray, bias=None, act: str = "none", residual=None, out: str = "f32", lib=None) -> np.ndarray:
    """The fused epilogue applied to a binary32 result Y [M, N]: float32 [M, N], or bf16 bits (uint16)."""
    Y = np.ascontiguousarray(Y, dtype=np.float32)
    M, N = Y.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    r = None if residual is None else np.ascontiguousarray(residual, dtype=np.float32)
    assert b is None or b.shape == (N,)
    assert r is None or r.shape == (M, N)
    o = np.empty((M, N), dtype=np.uint16 if out == "bf16" else np.float32)
    (lib or load()).oracle_epilogue(_ptr(Y), N, M, N, None if b is None else _ptr(b), ACTS[act],
                                    None if r is None else _ptr(r), N, 1 if out == "bf16" else 0, _ptr(o), N)
    return o


def ep_exp(x: float, lib=None) -> float:
    return float((lib or load()).oracle_ep_exp(float(x)))


def gemm_mfma(A: np.ndarray, W: np.ndarray, threads: int = 1, lib=None) -> np.ndarray:
    """Bit model of the matrix-core product (A [M, K], W [K, N] bf16 bits) -> float32 [M, N].

    Finite operands only: an exponent field of all ones is read as a number, so outputs that meet an Inf or
    NaN operand are not modelled (IEEE arithmetic fixes their class, NaN or an infinity, in any order)."""
    A = np.ascontiguousarray(A, dtype=np.uint16)
    W = np.ascontiguousarray(W, dtype=np.uint16)
    assert A.ndim == 2 and W.ndim == 2 and A.shape[1] == W.shape[0], (A.shape, W.shape)
    M, K = A.shape
    N = W.shape[1]
    out = np.empty((M, N), dtype=np.float32)
    fn = (lib or load()).oracle_gemm_mfma

    def run(r0, r1):
        if r1 > r0 and N > 0:
            fn(_ptr(A[r0:]), K, _ptr(W), N, _ptr(out[r0:]), N, r1 - r0, N, K)

    if threads <= 1 or M < 2:
        run(0, M)
    else:
        step = (M + threads - 1) // threads
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda r0: run(r0, min(M, r0 + step)), range(0, M, step)))
    return out


def gemv_tree(x: np.ndarray, WT: np.ndarray, threads: int = 1, lib=None) -> np.ndarray:
    """The tree-ordered GEMV: x [M, K] bf16 bits, WT [N, K] bf16 bits (W transposed) -> float32 [M, N].

    ``threads > 1`` splits the outputs' n range over threads; every output is computed whole by one
    call, so the bytes equal a single-threaded run."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    WT = np.ascontiguousarray(WT, dtype=np.uint16)
    assert x.ndim == 2 and WT.ndim == 2 and x.shape[1] == WT.shape[1], (x.shape, WT.shape)
    M, K = x.shape
    N = WT.shape[0]
    out = np.empty((M, N), dtype=np.float32)
    fn = (lib or load()).oracle_gemv_tree

    def run(n0, n1):
        if n1 > n0 and M > 0:
            fn(_ptr(x), K, _ptr(WT[n0:]), K, _ptr(out[:, n0:]), N, M, n1 - n0, K)

    if threads <= 1 or N < 2:
        run(0, N)
    else:
        step = (N + threads - 1) // threads
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda n0: run(n0, min(N, n0 + step)), range(0, N, step)))
    return out


def freivalds_prepare(W: np.ndarray, r: np.ndarray):
    """(s, q, a) K-vectors in float64 for matrix W [K, N] and signs r (int8, length N)."""
    W = np.ascontiguousarray(W, dtype=np.uint16)
    r = np.ascontiguousarray(r, dtype=np.int8)
    K, N = W.shape
    assert r.shape == (N,)
    s, q, a = (np.empty(K, dtype=np.float64) for _ in range(3))
    load().oracle_freivalds_prepare(_ptr(W), N, K, N, _ptr(r), _ptr(s), _ptr(q), _ptr(a))
    return s, q, a


def freivalds_check(prep, r: np.ndarray, x: np.ndarray, y: np.ndarray, c_f: float = 0.125):
    """Returns (accept: bool, rho, sigma, tau, bound) for one row x (bf16, K) and y (f32, N)."""
    s, q, a = prep
    x = np.ascontiguousarray(x, dtype=np.uint16)
    y = np.ascontiguousarray(y, dtype=np.float32)
    r = np.ascontiguousarray(r, dtype=np.int8)
    out = np.empty(4, dtype=np.float64)
    ok = load().oracle_freivalds_check(_ptr(s), _ptr(q), _ptr(a), _ptr(r), s.shape[0], y.shape[0],
                                       _ptr(x), _ptr(y), float(c_f), _ptr(out))
    return bool(ok), float(out[0]), float(out[1]), float(out[2]), float(out[3])
