"""Batch-invariant matrix multiply for MI355X (gfx950): Python binding.

Thin ctypes marshalling over the C-ABI in ``include/ggo.h``: every function
takes torch tensors (device memory and streams come from torch), checks
shapes and dtypes, and passes raw pointers, strides and the current HIP
stream to ``libggo.so``. All arithmetic runs in the library's HIP kernels
(the Freivalds certificate runs in the library's host code). If the library
is missing the import fails; there is no fallback.

bfloat16 operands are ``torch.bfloat16`` tensors (or int16/uint16 tensors
holding the bit patterns); results are ``torch.float32``.
"""
from __future__ import annotations

import ctypes as ct
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libggo.so")

GGO_BF16, GGO_F32 = 0, 1
GEMV_MAX_M = 16
MAX_PROBLEMS = 16


class GGOError(RuntimeError):
    pass


class Epilogue(ct.Structure):
    """Mirror of ``ggo_epilogue``."""
    _fields_ = [("bias", ct.c_void_p), ("residual", ct.c_void_p), ("ldr", ct.c_int64),
                ("act", ct.c_int), ("out_dtype", ct.c_int)]


ACTS = {"none": 0, "relu": 1, "silu": 2, "gelu_tanh": 3}


class CertStats(ct.Structure):
    """Mirror of ``ggo_cert_stats``."""
    _fields_ = [("submitted", ct.c_int64), ("checked", ct.c_int64), ("failed", ct.c_int64),
                ("max_honest_ratio", ct.c_double), ("check_seconds", ct.c_double), ("copy_error", ct.c_int),
                ("wait_seconds", ct.c_double), ("submit_wait_seconds", ct.c_double), ("submit_seconds", ct.c_double)]


class Problem(ct.Structure):
    """Mirror of ``ggo_problem``."""
    _fields_ = [("A", ct.c_void_p), ("W", ct.c_void_p), ("C", ct.c_void_p),
                ("lda", ct.c_int64), ("ldw", ct.c_int64), ("ldc", ct.c_int64),
                ("batch", ct.c_int64),
                ("stride_a", ct.c_int64), ("stride_w", ct.c_int64), ("stride_c", ct.c_int64),
                ("M", ct.c_int64), ("N", ct.c_int64), ("K", ct.c_int64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() (hipcc for gfx950) first")
    # torch first: its HIP runtime is then the one libggo.so binds to, so device memory, streams and
    # launches all live in one runtime (loading the library first brings in a second one)
    import torch  # noqa: F401
    lib = ct.CDLL(LIB_PATH)
    P, I64, I = ct.c_void_p, ct.c_int64, ct.c_int
    lib.gemm_ordered.argtypes = [P, I, I64, P, I64, P, I64, I64, I64, I64, P]
    lib.gemm_ordered_grouped.argtypes = [ct.POINTER(Problem), I64, I, P]
    lib.gemv_ordered.argtypes = [P, I64, P, I64, P, I64, I64, I64, I64, P]
    lib.gemv_ordered_wt.argtypes = [P, I64, P, I64, P, I64, I64, I64, I64, P]
    lib.gemv_tree.argtypes = [P, I64, P, I64, P, I64, I64, I64, I64, P]
    lib.gemv_tree_ep.argtypes = [P, I64, P, I64, ct.POINTER(Epilogue), P, I64, I64, I64, I64, P]
    lib.gemm_mfma_invariant_ep.argtypes = [P, I64, P, I64, ct.POINTER(Epilogue), P, I64, I64, I64, I64, P]
    lib.gemm_mfma_invariant.argtypes = [P, I64, P, I64, P, I64, I64, I64, I64, P]
    lib.ggo_test_gemm_mfma_tile128.argtypes = [P, I64, P, I64, P, I64, I64, I64, I64, P]
    lib.gemm_mfma_invariant_wt.argtypes = [P, I64, P, I64, P, I64, I64, I64, I64, P]
    lib.gemv_mfma_invariant.argtypes = [P, I64, P, I64, P, I64, I64, I64, I64, P]
    lib.gemv_mfma_invariant_ep.argtypes = [P, I64, P, I64, ct.POINTER(Epilogue), P, I64, I64, I64, I64, P]
    PP = ct.POINTER(ct.c_void_p)
    lib.ggo_test_gemv_instance.argtypes = [I, I, I, P, I64, P, I64, P, I64, I64, I64, I64, P]
    lib.ggo_test_gemm_ordered_tile.argtypes = [I, P, I, I64, P, I64, P, I64, I64, I64, I64, P]
    lib.ggo_test_gemm_mfma_tile.argtypes = [I, P, I64, P, I64, P, I64, I64, I64, I64, P]
    lib.freivalds_prepare.argtypes = [P, I64, I64, I64, ct.c_uint64, PP]
    lib.freivalds_check.argtypes = [P, P, P, ct.c_double, P]
    lib.freivalds_signs.argtypes = [P, P]
    lib.freivalds_free.argtypes = [P]
    lib.freivalds_free.restype = None
    lib.freivalds_prepare_signs.argtypes = [P, I64, I64, I64, P, P, P, P]
    lib.freivalds_check_signs.argtypes = [P, P, P, P, I64, I64, P, P, ct.c_double, P]
    lib.ggo_cert_create.argtypes = [I64, I64, I64, I, ct.c_double, PP]
    lib.ggo_cert_create_host.argtypes = [I64, I64, I64, I, ct.c_double, PP]
    lib.ggo_cert_add_matrix.argtypes = [P, P, I64, I, I64, I64, P, I64, ct.POINTER(I)]
    lib.ggo_cert_submit.argtypes = [P, I, P, P, I64, P]
    lib.ggo_cert_submit_host.argtypes = [P, I, P, P, I64]
    lib.ggo_cert_submit_rows.argtypes = [P, I64, P, P, P, I64, P]
    lib.ggo_cert_drain.argtypes = [P, ct.POINTER(CertStats)]
    lib.ggo_cert_failures.argtypes = [P, P, P, I64]
    lib.ggo_cert_failures.restype = I64
    lib.ggo_cert_destroy.argtypes = [P]
    lib.ggo_cert_destroy.restype = None
    for f in ("ggo_cert_create", "ggo_cert_create_host", "ggo_cert_add_matrix", "ggo_cert_submit",
              "ggo_cert_submit_rows", "ggo_cert_submit_host", "ggo_cert_drain"):
        getattr(lib, f).restype = I
    lib.ggo_build_info.restype = ct.c_char_p
    lib.ggo_last_error.restype = ct.c_char_p
    for f in ("gemm_ordered", "gemm_ordered_grouped", "gemv_ordered", "gemv_ordered_wt", "gemv_tree", "gemv_tree_ep",
              "gemm_mfma_invariant_ep", "gemm_mfma_invariant",
              "ggo_test_gemm_mfma_tile128", "ggo_test_gemv_instance", "ggo_test_gemm_ordered_tile",
              "ggo_test_gemm_mfma_tile", "gemm_mfma_invariant_wt", "gemv_mfma_invariant",
              "gemv_mfma_invariant_ep", "freivalds_prepare", "freivalds_check", "freivalds_signs",
              "freivalds_prepare_signs", "freivalds_check_signs"):
        getattr(lib, f).restype = I
    return lib


lib = _load()

EXPORTS = ("gemm_ordered", "gemm_ordered_grouped", "gemv_ordered", "gemv_ordered_wt", "gemv_tree", "gemv_tree_ep",
           "gemm_mfma_invariant_ep", "gemm_mfma_invariant",
           "gemm_mfma_invariant_wt", "gemv_mfma_invariant", "gemv_mfma_invariant_ep",
           "ggo_test_gemm_mfma_tile128", "ggo_test_gemv_instance", "ggo_test_gemm_ordered_tile",
           "ggo_test_gemm_mfma_tile", "freivalds_prepare", "freivalds_check",
           "freivalds_signs", "freivalds_free", "freivalds_prepare_signs", "freivalds_check_signs",
           "ggo_build_info", "ggo_last_error",
           "ggo_cert_create", "ggo_cert_create_host", "ggo_cert_add_matrix", "ggo_cert_submit", "ggo_cert_submit_rows",
           "ggo_cert_submit_host",
           "ggo_cert_drain", "ggo_cert_failures", "ggo_cert_destroy")


def build_info() -> str:
    return lib.ggo_build_info().decode()


def _raise(rc: int, fn: str):
    if rc < 0:
        raise GGOError(f"{fn} failed ({rc}): {lib.ggo_last_error().decode()}")


def _torch():
    import torch
    return torch


def _is_bf16(t) -> bool:
    torch = _torch()
    return t.dtype in (torch.bfloat16, torch.int16) or str(t.dtype) == "torch.uint16"


def _rowmajor(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got {tuple(t.shape)}")
    if t.shape[0] > 0 and t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along its last axis")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return max(t.stride(0), t.shape[1])


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ct.c_void_p(s.cuda_stream)


def _out(C, M, N, like):
    torch = _torch()
    if C is None:
        return torch.empty((M, N), dtype=torch.float32, device=like.device)
    if C.dtype != torch.float32 or tuple(C.shape) != (M, N):
        raise ValueError(f"C must be float32 [{M}, {N}]")
    return C


def gemm_ordered(A, W, C=None, stream=None):
    """C = A W under the order contract (A bf16 or float32, W bf16, C float32)."""
    torch = _torch()
    lda, ldw = _rowmajor(A, "A"), _rowmajor(W, "W")
    M, K = A.shape
    if W.shape[0] != K or not _is_bf16(W):
        raise ValueError("W must be bf16 [K, N]")
    N = W.shape[1]
    if _is_bf16(A):
        ad = GGO_BF16
    elif A.dtype == torch.float32:
        ad = GGO_F32
    else:
        raise ValueError(f"A must be bf16 or float32, got {A.dtype}")
    C = _out(C, M, N, A)
    ldc = _rowmajor(C, "C") if M and N else N
    _raise(lib.gemm_ordered(A.data_ptr(), ad, lda, W.data_ptr(), ldw, C.data_ptr(), ldc, M, N, K, _stream(stream)),
           "gemm_ordered")
    return C


ORDERED_TILES = {"64x64": 0, "16x16": 1, "64x32": 2}


def test_gemm_ordered_tile(tile, A, W, C=None, stream=None):
    """Test hook: gemm_ordered on the chosen tile ('64x64', '64x32' or '16x16'); must give gemm_ordered's
    bits."""
    torch = _torch()
    lda, ldw = _rowmajor(A, "A"), _rowmajor(W, "W")
    M, K = A.shape
    if W.shape[0] != K or not _is_bf16(W):
        raise ValueError("W must be bf16 [K, N]")
    N = W.shape[1]
    ad = GGO_BF16 if _is_bf16(A) else GGO_F32 if A.dtype == torch.float32 else None
    if ad is None:
        raise ValueError(f"A must be bf16 or float32, got {A.dtype}")
    C = _out(C, M, N, A)
    ldc = _rowmajor(C, "C") if M and N else N
    _raise(lib.ggo_test_gemm_ordered_tile(ORDERED_TILES[tile], A.data_ptr(), ad, lda, W.data_ptr(), ldw, C.data_ptr(),
                                          ldc, M, N, K, _stream(stream)), "ggo_test_gemm_ordered_tile")
    return C


def gemm_ordered_grouped(problems, stream=None):
    """problems: list of (A, W, C) with A [b, M, K] (bf16 or float32, all the same), W [b, K, N] bf16,
    C [b, M, N] float32 (3-D, or 2-D for b = 1). One launch; each output has gemm_ordered's bits."""
    torch = _torch()
    if not 1 <= len(problems) <= MAX_PROBLEMS:
        raise ValueError(f"1..{MAX_PROBLEMS} problems per launch")
    arr = (Problem * len(problems))()
    ad = None
    keep = []
    for i, (A, W, C) in enumerate(problems):
        A3, W3, C3 = (t if t.dim() == 3 else t.unsqueeze(0) for t in (A, W, C))
        b, M, K = A3.shape
        if W3.shape[0] != b or W3.shape[1] != K or C3.shape[0] != b or C3.shape[1] != M or C3.shape[2] != W3.shape[2]:
            raise ValueError("shape mismatch in grouped problem %d" % i)
        this = GGO_BF16 if _is_bf16(A3) else GGO_F32 if A3.dtype == torch.float32 else None
        if this is None or (ad is not None and this != ad) or not _is_bf16(W3) or C3.dtype != torch.float32:
            raise ValueError("dtype mismatch in grouped problem %d" % i)
        ad = this
        for t, nm in ((A3, "A"), (W3, "W"), (C3, "C")):
            if not t.is_cuda or (t.shape[2] > 1 and t.stride(2) != 1):
                raise ValueError(f"{nm} of problem {i} must be a device tensor with unit inner stride")
        arr[i] = Problem(A3.data_ptr(), W3.data_ptr(), C3.data_ptr(),
                         max(A3.stride(1), K), max(W3.stride(1), W3.shape[2]), max(C3.stride(1), C3.shape[2]),
                         b, A3.stride(0), W3.stride(0), C3.stride(0), M, W3.shape[2], K)
        keep.append((A3, W3, C3))
    _raise(lib.gemm_ordered_grouped(arr, len(problems), ad, _stream(stream)), "gemm_ordered_grouped")


def gemv_ordered(x, W, y=None, stream=None):
    """y = x W for x bf16 [M <= 16, K], W bf16 [K, N]: the same bits as gemm_ordered."""
    ldx, ldw = _rowmajor(x, "x"), _rowmajor(W, "W")
    M, K = x.shape
    if not (_is_bf16(x) and _is_bf16(W)) or W.shape[0] != K:
        raise ValueError("x and W must be bf16, W [K, N]")
    N = W.shape[1]
    y = _out(y, M, N, x)
    ldy = _rowmajor(y, "y") if M and N else N
    _raise(lib.gemv_ordered(x.data_ptr(), ldx, W.data_ptr(), ldw, y.data_ptr(), ldy, M, N, K, _stream(stream)),
           "gemv_ordered")
    return y


def gemv_ordered_wt(x, WT, y=None, stream=None):
    """gemv_ordered with the weight given transposed, WT bf16 [N, K] (k contiguous): the same order contract
    and bits. Needs 8-byte aligned operands with row strides and K multiples of 4."""
    ldx, ldwt = _rowmajor(x, "x"), _rowmajor(WT, "WT")
    M, K = x.shape
    if not (_is_bf16(x) and _is_bf16(WT)) or WT.shape[1] != K:
        raise ValueError("x and WT must be bf16, WT [N, K]")
    N = WT.shape[0]
    y = _out(y, M, N, x)
    ldy = _rowmajor(y, "y") if M and N else N
    _raise(lib.gemv_ordered_wt(x.data_ptr(), ldx, WT.data_ptr(), ldwt, y.data_ptr(), ldy, M, N, K, _stream(stream)),
           "gemv_ordered_wt")
    return y


def gemv_tree(x, WT, y=None, stream=None):
    """y = x W for x bf16 [M <= 16, K] and the weight given transposed, WT bf16 [N, K] (k contiguous):
    the tree order (8-k tiles dealt over 256 fused chains, count-up pairwise tree), bits independent of M."""
    ldx, ldwt = _rowmajor(x, "x"), _rowmajor(WT, "WT")
    M, K = x.shape
    if not (_is_bf16(x) and _is_bf16(WT)) or WT.shape[1] != K:
        raise ValueError("x and WT must be bf16, WT [N, K]")
    N = WT.shape[0]
    y = _out(y, M, N, x)
    ldy = _rowmajor(y, "y") if M and N else N
    _raise(lib.gemv_tree(x.data_ptr(), ldx, WT.data_ptr(), ldwt, y.data_ptr(), ldy, M, N, K, _stream(stream)),
           "gemv_tree")
    return y


def gemv_mfma_invariant(x, WT, y=None, stream=None):
    """y = x W for x bf16 [M <= 16, K] and the weight given transposed, WT bf16 [N, K], on the matrix cores:
    the bits of gemm_mfma_invariant(x, W) for every row and every M. Needs 16-byte aligned operands with
    row strides and K multiples of 8."""
    ldx, ldwt = _rowmajor(x, "x"), _rowmajor(WT, "WT")
    M, K = x.shape
    if not (_is_bf16(x) and _is_bf16(WT)) or WT.shape[1] != K:
        raise ValueError("x and WT must be bf16, WT [N, K]")
    N = WT.shape[0]
    y = _out(y, M, N, x)
    ldy = _rowmajor(y, "y") if M and N else N
    _raise(lib.gemv_mfma_invariant(x.data_ptr(), ldx, WT.data_ptr(), ldwt, y.data_ptr(), ldy, M, N, K,
                                   _stream(stream)), "gemv_mfma_invariant")
    return y


def gemv_mfma_invariant_ep(x, WT, bias=None, act="none", residual=None, out="f32", y=None, stream=None):
    """gemv_mfma_invariant followed, in the same kernel, by y = act(y + bias) + residual (fixed order), stored
    as float32 or bfloat16 (out='bf16')."""
    ldx, ldwt = _rowmajor(x, "x"), _rowmajor(WT, "WT")
    M, K = x.shape
    if not (_is_bf16(x) and _is_bf16(WT)) or WT.shape[1] != K:
        raise ValueError("x and WT must be bf16, WT [N, K]")
    N = WT.shape[0]
    e, y, keep = _epilogue(M, N, x, bias, act, residual, out, y)
    ldy = _rowmajor(y, "y") if M and N else N
    _raise(lib.gemv_mfma_invariant_ep(x.data_ptr(), ldx, WT.data_ptr(), ldwt, ct.byref(e), y.data_ptr(), ldy, M, N,
                                      K, _stream(stream)), "gemv_mfma_invariant_ep")
    return y


def _epilogue(M, N, like, bias, act, residual, out, y):
    """Build the ggo_epilogue and the output tensor (float32, or bfloat16 for out='bf16')."""
    torch = _torch()
    if act not in ACTS:
        raise ValueError(f"act must be one of {sorted(ACTS)}")
    if out not in ("f32", "bf16"):
        raise ValueError("out must be 'f32' or 'bf16'")
    keep = []
    e = Epilogue(None, None, 0, ACTS[act], GGO_BF16 if out == "bf16" else GGO_F32)
    if bias is not None:
        if bias.dtype != torch.float32 or tuple(bias.shape) != (N,) or not bias.is_cuda or (N > 1 and bias.stride(0) != 1):
            raise ValueError(f"bias must be a contiguous float32 device tensor [{N}]")
        e.bias = bias.data_ptr()
        keep.append(bias)
    if residual is not None:
        if residual.dtype != torch.float32 or tuple(residual.shape) != (M, N):
            raise ValueError(f"residual must be float32 [{M}, {N}]")
        e.residual = residual.data_ptr()
        e.ldr = _rowmajor(residual, "residual") if M and N else N
        keep.append(residual)
    want = torch.bfloat16 if out == "bf16" else torch.float32
    if y is None:
        y = torch.empty((M, N), dtype=want, device=like.device)
    elif y.dtype != want or tuple(y.shape) != (M, N):
        raise ValueError(f"output must be {want} [{M}, {N}]")
    return e, y, keep


def gemv_tree_ep(x, WT, bias=None, act="none", residual=None, out="f32", y=None, stream=None):
    """gemv_tree followed, in the same kernel, by y = act(y + bias) + residual (fixed order), stored as
    float32 or bfloat16 (out='bf16')."""
    ldx, ldwt = _rowmajor(x, "x"), _rowmajor(WT, "WT")
    M, K = x.shape
    if not (_is_bf16(x) and _is_bf16(WT)) or WT.shape[1] != K:
        raise ValueError("x and WT must be bf16, WT [N, K]")
    N = WT.shape[0]
    e, y, keep = _epilogue(M, N, x, bias, act, residual, out, y)
    ldy = _rowmajor(y, "y") if M and N else N
    _raise(lib.gemv_tree_ep(x.data_ptr(), ldx, WT.data_ptr(), ldwt, ct.byref(e), y.data_ptr(), ldy, M, N, K,
                            _stream(stream)), "gemv_tree_ep")
    return y


def gemm_mfma_invariant_ep(A, W, bias=None, act="none", residual=None, out="f32", C=None, stream=None):
    """gemm_mfma_invariant followed, in the same kernel, by C = act(C + bias) + residual (fixed order),
    stored as float32 or bfloat16 (out='bf16')."""
    lda, ldw = _rowmajor(A, "A"), _rowmajor(W, "W")
    M, K = A.shape
    if not (_is_bf16(A) and _is_bf16(W)) or W.shape[0] != K:
        raise ValueError("A and W must be bf16, W [K, N]")
    N = W.shape[1]
    e, C, keep = _epilogue(M, N, A, bias, act, residual, out, C)
    ldc = _rowmajor(C, "C") if M and N else N
    _raise(lib.gemm_mfma_invariant_ep(A.data_ptr(), lda, W.data_ptr(), ldw, ct.byref(e), C.data_ptr(), ldc, M, N, K,
                                      _stream(stream)), "gemm_mfma_invariant_ep")
    return C


def _mfma(fn, A, W, C, stream):
    lda, ldw = _rowmajor(A, "A"), _rowmajor(W, "W")
    M, K = A.shape
    if not (_is_bf16(A) and _is_bf16(W)) or W.shape[0] != K:
        raise ValueError("A and W must be bf16, W [K, N]")
    N = W.shape[1]
    C = _out(C, M, N, A)
    ldc = _rowmajor(C, "C") if M and N else N
    _raise(getattr(lib, fn)(A.data_ptr(), lda, W.data_ptr(), ldw, C.data_ptr(), ldc, M, N, K, _stream(stream)), fn)
    return C


def gemm_mfma_invariant(A, W, C=None, stream=None):
    """C = A W on the matrix cores, bits independent of M (A, W bf16; C float32)."""
    return _mfma("gemm_mfma_invariant", A, W, C, stream)


def gemm_mfma_invariant_wt(A, WT, C=None, stream=None):
    """C = A W with W given transposed (WT [N, K] bf16, k contiguous): the bits of gemm_mfma_invariant(A, W)."""
    lda, ldwt = _rowmajor(A, "A"), _rowmajor(WT, "WT")
    M, K = A.shape
    if not (_is_bf16(A) and _is_bf16(WT)) or WT.shape[1] != K:
        raise ValueError("A and WT must be bf16, WT [N, K]")
    N = WT.shape[0]
    C = _out(C, M, N, A)
    ldc = _rowmajor(C, "C") if M and N else N
    _raise(lib.gemm_mfma_invariant_wt(A.data_ptr(), lda, WT.data_ptr(), ldwt, C.data_ptr(), ldc, M, N, K,
                                      _stream(stream)), "gemm_mfma_invariant_wt")
    return C


def test_gemm_mfma_tile128(A, W, C=None, stream=None):
    """Test hook: the same descriptor on the 128x128 tile instance (must give the same bits)."""
    return _mfma("ggo_test_gemm_mfma_tile128", A, W, C, stream)


MFMA_TILES = {"256x128": 0, "128x128": 1, "64x64": 2, "256x256": 3, "128x128_lds": 4, "64x128_lds": 5}


def test_gemm_mfma_tile(tile, A, W, C=None, stream=None):
    """Test hook: gemm_mfma_invariant on the chosen tile instance (a key of MFMA_TILES); must
    give gemm_mfma_invariant's bits."""
    lda, ldw = _rowmajor(A, "A"), _rowmajor(W, "W")
    M, K = A.shape
    if not (_is_bf16(A) and _is_bf16(W)) or W.shape[0] != K:
        raise ValueError("A and W must be bf16, W [K, N]")
    N = W.shape[1]
    C = _out(C, M, N, A)
    ldc = _rowmajor(C, "C") if M and N else N
    _raise(lib.ggo_test_gemm_mfma_tile(MFMA_TILES[tile], A.data_ptr(), lda, W.data_ptr(), ldw, C.data_ptr(), ldc,
                                       M, N, K, _stream(stream)), "ggo_test_gemm_mfma_tile")
    return C


GEMV_KINDS = {"tree": 0, "ordered": 1, "ordered_wt": 2, "mfma": 3}


def test_gemv_instance(kind, rows, form, x, W, y=None, stream=None):
    """Test hook: the decode GEMV `kind` ('tree', 'ordered', 'ordered_wt', 'mfma') run by a chosen kernel
    instance (rows of x staged per workgroup, and the form; see ggo_test_gemv_instance) instead of the one
    its entry point picks from M. W is W [K, N] for 'ordered', else W^T [N, K]. Must give the entry
    point's bits."""
    ldx, ldw = _rowmajor(x, "x"), _rowmajor(W, "W")
    M, K = x.shape
    transposed = kind != "ordered"
    if not (_is_bf16(x) and _is_bf16(W)) or (W.shape[1] if transposed else W.shape[0]) != K:
        raise ValueError("x and W must be bf16 with matching K")
    N = W.shape[0] if transposed else W.shape[1]
    y = _out(y, M, N, x)
    ldy = _rowmajor(y, "y") if M and N else N
    _raise(lib.ggo_test_gemv_instance(GEMV_KINDS[kind], rows, form, x.data_ptr(), ldx, W.data_ptr(), ldw,
                                      y.data_ptr(), ldy, M, N, K, _stream(stream)), "ggo_test_gemv_instance")
    return y


def _np(a, dtype):
    if hasattr(a, "detach"):
        a = a.detach().cpu()
        if str(a.dtype) == "torch.bfloat16":
            a = a.view(_torch().int16)
        a = a.numpy()
    return np.ascontiguousarray(a).view(dtype) if np.asarray(a).dtype.itemsize == np.dtype(dtype).itemsize \
        else np.ascontiguousarray(a, dtype=dtype)


class Freivalds:
    """Handle of the float Freivalds certificate for one matrix (freivalds_prepare / freivalds_check /
    freivalds_free): W [K, N] host bf16 bits; the N signs are drawn inside the library from `seed`."""

    def __init__(self, W, seed: int):
        W = np.ascontiguousarray(_np(W, np.uint16))
        self.K, self.N = W.shape
        h = ct.c_void_p()
        _raise(lib.freivalds_prepare(W.ctypes.data, self.N, self.K, self.N, ct.c_uint64(seed & (2 ** 64 - 1)),
                                     ct.byref(h)), "freivalds_prepare")
        self.h = h

    def check(self, x, y, c_f: float = 0.125):
        """(accept, rho, sigma, tau, bound) for one host row x (bf16 bits, K) and y (float32, N)."""
        x = np.ascontiguousarray(_np(x, np.uint16)).reshape(-1)
        y = np.ascontiguousarray(_np(y, np.float32)).reshape(-1)
        if x.size != self.K or y.size != self.N:
            raise ValueError(f"x must hold {self.K} and y {self.N} elements")
        out = np.empty(4, dtype=np.float64)
        rc = lib.freivalds_check(self.h, x.ctypes.data, y.ctypes.data, float(c_f), out.ctypes.data)
        _raise(rc, "freivalds_check")
        return bool(rc), float(out[0]), float(out[1]), float(out[2]), float(out[3])

    def signs(self) -> np.ndarray:
        r = np.empty(self.N, dtype=np.int8)
        _raise(lib.freivalds_signs(self.h, r.ctypes.data), "freivalds_signs")
        return r

    def close(self):
        if self.h:
            lib.freivalds_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def freivalds_prepare(W, seed: int) -> Freivalds:
    """freivalds_prepare: the certificate handle of W [K, N] (host bf16 bits) with signs drawn from seed."""
    return Freivalds(W, seed)


def freivalds_prepare_signs(W, r):
    """Host precompute (s, q, a) for W [K, N] (bf16 bits, host) and caller-drawn signs r (N, +-1)."""
    W = _np(W, np.uint16)
    r = np.ascontiguousarray(r, dtype=np.int8)
    K, N = W.shape
    s, q, a = (np.empty(K, dtype=np.float64) for _ in range(3))
    _raise(lib.freivalds_prepare_signs(W.ctypes.data, N, K, N, r.ctypes.data, s.ctypes.data, q.ctypes.data,
                                       a.ctypes.data), "freivalds_prepare_signs")
    return s, q, a


def freivalds_check_signs(prep, r, x, y, c_f: float = 0.125):
    """(accept, rho, sigma, tau, bound) for one host row x (bf16 bits, K) and y (float32, N)."""
    s, q, a = prep
    x = _np(x, np.uint16).reshape(-1)
    y = _np(y, np.float32).reshape(-1)
    r = np.ascontiguousarray(r, dtype=np.int8)
    out = np.empty(4, dtype=np.float64)
    rc = lib.freivalds_check_signs(s.ctypes.data, q.ctypes.data, a.ctypes.data, r.ctypes.data, s.shape[0],
                                   y.shape[0], x.ctypes.data, y.ctypes.data, float(c_f), out.ctypes.data)
    _raise(rc, "freivalds_check_signs")
    return bool(rc), float(out[0]), float(out[1]), float(out[2]), float(out[3])


class CertEngine:
    """The certificate engine of ``ggo_cert_*``: register matrices (host bf16 weights and t sign vectors
    each), submit sampled output rows from the device (asynchronous copies on the engine's own stream)
    or from the host, drain, and read the failures."""

    def __init__(self, max_K, max_N, slots=64, workers=2, c_f=0.125, host_only=False):
        h = ct.c_void_p()
        create = lib.ggo_cert_create_host if host_only else lib.ggo_cert_create
        rc = create(max_K, max_N, slots, workers, float(c_f), ct.byref(h))
        if rc < 0:
            raise GGOError(f"ggo_cert_create failed ({rc})")
        self.h = h
        self.K = {}
        self.N = {}

    def add_matrix(self, W, r, transposed=False):
        """W: host bf16 bits, [K, N] (or [N, K] with transposed=True); r: [t, N] signs (+1/-1)."""
        W = _np(W, np.uint16)
        W = np.ascontiguousarray(W)
        r = np.ascontiguousarray(np.atleast_2d(r), dtype=np.int8)
        N, K = (W.shape if transposed else W.shape[::-1])
        if r.shape[1] != N:
            raise ValueError(f"r must have {N} columns")
        mid = ct.c_int()
        _raise(lib.ggo_cert_add_matrix(self.h, W.ctypes.data, W.shape[1], int(transposed), K, N, r.ctypes.data,
                                       r.shape[0], ct.byref(mid)), "ggo_cert_add_matrix")
        self.K[mid.value], self.N[mid.value] = K, N
        return mid.value

    def submit(self, mid, x_row, y_row, token, stream=None):
        """x_row: device bf16 [K], y_row: device float32 [N] (contiguous)."""
        if x_row.numel() != self.K[mid] or y_row.numel() != self.N[mid] or not x_row.is_contiguous() \
                or not y_row.is_contiguous():
            raise ValueError("x_row / y_row must be contiguous rows of the matrix's K / N")
        _raise(lib.ggo_cert_submit(self.h, mid, x_row.data_ptr(), y_row.data_ptr(), int(token), _stream(stream)),
               "ggo_cert_submit")

    def submit_rows(self, mids, x_rows, y_rows, token, stream=None):
        """Several rows (<= 16) of one token in one call: one gather launch on the engine's stream."""
        n = len(mids)
        for mid, x, y in zip(mids, x_rows, y_rows):
            if x.numel() != self.K[mid] or y.numel() != self.N[mid] or not x.is_contiguous() or not y.is_contiguous():
                raise ValueError("x / y must be contiguous rows of the matrix's K / N")
        ids = (ct.c_int * n)(*mids)
        xs = (ct.c_void_p * n)(*[x.data_ptr() for x in x_rows])
        ys = (ct.c_void_p * n)(*[y.data_ptr() for y in y_rows])
        _raise(lib.ggo_cert_submit_rows(self.h, n, ids, xs, ys, int(token), _stream(stream)), "ggo_cert_submit_rows")

    def submit_host(self, mid, x_row, y_row, token):
        x = np.ascontiguousarray(_np(x_row, np.uint16)).reshape(-1)
        y = np.ascontiguousarray(_np(y_row, np.float32)).reshape(-1)
        if x.size != self.K[mid] or y.size != self.N[mid]:
            raise ValueError("row sizes do not match the matrix")
        _raise(lib.ggo_cert_submit_host(self.h, mid, x.ctypes.data, y.ctypes.data, int(token)), "ggo_cert_submit_host")

    def drain(self):
        st = CertStats()
        _raise(lib.ggo_cert_drain(self.h, ct.byref(st)), "ggo_cert_drain")
        return {f: getattr(st, f) for f, _ in CertStats._fields_}

    def failures(self, cap=1 << 16):
        toks = np.empty(cap, dtype=np.int64)
        mats = np.empty(cap, dtype=np.int32)
        n = lib.ggo_cert_failures(self.h, toks.ctypes.data, mats.ctypes.data, cap)
        n = min(n, cap)
        return list(zip(toks[:n].tolist(), mats[:n].tolist()))

    def close(self):
        if self.h:
            lib.ggo_cert_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
