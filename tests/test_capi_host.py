"""The C-ABI library on the host: it loads, exports every entry point the header
declares, reports its sources, rejects bad arguments, and its host-side
Freivalds certificate agrees with the oracle's. No GPU work is launched."""
import ctypes as ct
import json
import os
import re

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ggo.h")


@pytest.fixture(scope="module")
def g():
    import gemv_gemm_ordered_amd as g
    return g


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)) - {"if", "defined"})


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("gemm_ordered", "gemm_ordered_grouped", "gemv_ordered", "gemv_tree", "gemm_mfma_invariant",
              "freivalds_prepare", "freivalds_check", "ggo_build_info", "ggo_last_error"):
        assert n in names, names


def test_library_exports_every_declared_symbol(g):
    lib = ct.CDLL(g.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in ggo.h but not exported"
    assert set(declared_functions()) == set(g.EXPORTS)


def test_build_info_names_current_sources(g):
    from gemv_gemm_ordered_amd import build as gb
    info = json.loads(g.build_info())
    assert info["arch"] == "gfx950"
    assert "-ffp-contract=off" in info["flags"] and "-packed-fp32-ops" in info["flags"]
    for src, digest in info["sources"].items():
        assert digest == gb._sha(os.path.join(gb.CSRC, src)), f"library is stale for {src}: rebuild"


def test_bad_arguments_are_rejected_without_touching_the_gpu(g):
    lib = g.lib
    null = None
    # negative sizes, bad dtype, short strides, over-large gemv M
    assert lib.gemm_ordered(null, 0, 8, null, 8, null, 8, -1, 8, 8, null) == -1
    assert b"negative" in lib.ggo_last_error()
    assert lib.gemm_ordered(1, 7, 8, 1, 8, 1, 8, 4, 8, 8, null) == -1
    assert lib.gemm_ordered(1, 0, 4, 1, 8, 1, 8, 4, 8, 8, null) == -1     # lda < K
    assert lib.gemm_ordered(null, 0, 8, 1, 8, 1, 8, 4, 8, 8, null) == -1  # null A
    assert lib.gemv_ordered(1, 8, 1, 8, 1, 8, 17, 8, 8, null) == -2
    assert lib.gemv_tree(1, 8, 1, 8, 1, 8, 17, 8, 8, null) == -2           # M > 16
    assert lib.gemv_tree(1, 8, 1, 4, 1, 8, 4, 8, 8, null) == -1            # ldwt < K
    assert lib.gemv_tree(1, 8, 1, 8, 1, 4, 4, 8, 8, null) == -1            # ldy < N
    assert lib.gemv_tree(1, 1 << 30, 1, 1 << 30, 1, 8, 1, 8, 1 << 30, null) == -2   # K too large
    assert lib.gemm_mfma_invariant(1, 8, 1, 4, 1, 8, 4, 8, 8, null) == -1  # ldw < N
    # matrix-core GEMV and the W^T ordered GEMV: M > 16, short strides, alignment, K multiples, null pointers
    for f in (lib.gemv_mfma_invariant, lib.gemv_ordered_wt):
        assert f(16, 8, 16, 8, 16, 8, 17, 8, 8, null) == -2                 # M > 16
        assert f(16, 8, 16, 4, 16, 8, 4, 8, 8, null) == -1                 # ldwt < K
        assert f(16, 8, 16, 8, 16, 4, 4, 8, 8, null) == -1                  # ldy < N
        assert f(null, 8, 16, 8, 16, 8, 4, 8, 8, null) == -1                # null x
        assert f(18, 8, 16, 8, 16, 8, 4, 8, 8, null) == -2                  # x misaligned (2 bytes)
        assert f(16, 8, 16, 8, 16, 8, 4, 8, 6, null) == -2                  # K % 4 != 0 (and % 8)
    assert lib.gemv_mfma_invariant(16, 12, 16, 12, 16, 8, 4, 8, 12, null) == -2   # K % 8 != 0
    assert lib.gemv_mfma_invariant(16, 1 << 29, 16, 1 << 29, 16, 8, 1, 8, 1 << 29, null) == -2   # K too large
    assert b"too large" in lib.ggo_last_error()
    assert lib.gemm_ordered_grouped(null, 1, 0, null) == -1
    arr = (g.Problem * 1)()
    assert lib.gemm_ordered_grouped(arr, 17, 0, null) == -1
    # empty problems are valid and launch nothing
    assert lib.gemm_ordered(null, 0, 8, null, 8, null, 8, 0, 8, 8, null) == 0
    assert lib.gemv_ordered(null, 8, null, 8, null, 8, 0, 8, 8, null) == 0
    assert lib.gemv_tree(null, 8, null, 8, null, 8, 0, 8, 8, null) == 0
    assert lib.gemv_tree(null, 8, null, 8, null, 8, 3, 0, 8, null) == 0
    assert lib.gemm_mfma_invariant(null, 8, null, 8, null, 8, 5, 0, 8, null) == 0
    assert lib.gemv_mfma_invariant(null, 8, null, 8, null, 8, 0, 8, 8, null) == 0
    assert lib.gemv_ordered_wt(null, 8, null, 8, null, 8, 3, 0, 8, null) == 0
    assert lib.ggo_last_error() == b""


def test_freivalds_host_matches_oracle(g):
    x, W, r = synth.decode_gemv(2, 4, k=512, n=768)
    y = oracle.gemm_ordered(x, W)
    prep_g = g.freivalds_prepare(W, r)
    prep_o = oracle.freivalds_prepare(W, r)
    for a, b in zip(prep_g, prep_o):
        assert np.array_equal(a, b)
    for m in range(4):
        yb = y[m].copy()
        if m == 3:
            yb[100] += np.float32(0.005)
        res_g = g.freivalds_check(prep_g, r, x[m], yb, 0.125)
        res_o = oracle.freivalds_check(prep_o, r, x[m], yb, 0.125)
        assert res_g[0] == res_o[0] == (m != 3)
        assert np.allclose(res_g[1:], res_o[1:], rtol=1e-12, atol=1e-15)


def test_freivalds_rejects_bad_signs(g):
    W = np.zeros((4, 4), dtype=np.uint16)
    with pytest.raises(g.GGOError):
        g.freivalds_prepare(W, np.array([1, 0, -1, 1], dtype=np.int8))
