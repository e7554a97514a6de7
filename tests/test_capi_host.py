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
              "freivalds_prepare", "freivalds_check", "freivalds_free", "ggo_build_info", "ggo_last_error",
              "ggo_test_gemv_instance"):
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
    # size limits of the ordered GEMVs (32-bit offsets inside a stage or slab) and of every size argument
    assert lib.gemv_ordered(16, 8, 16, 1 << 25, 16, 8, 1, 8, 8, null) == -2             # ldw past the stage range
    assert b"too large" in lib.ggo_last_error()
    assert lib.gemv_ordered(16, 1 << 30, 16, 8, 16, 8, 1, 8, 1 << 30, null) == -2       # K >= 2^30
    assert b"too large" in lib.ggo_last_error()
    assert lib.gemv_ordered_wt(16, 8, 16, 1 << 27, 16, 8, 1, 8, 8, null) == -2          # ldwt past the slab range
    assert b"too large" in lib.ggo_last_error()
    assert lib.gemm_ordered(16, 0, 8, 16, 8, 16, 8, 1 << 31, 8, 8, null) == -2          # M > 2^31 - 1
    assert b"2^31-1" in lib.ggo_last_error()
    assert lib.gemm_mfma_invariant(16, 1 << 31, 16, 8, 16, 8, 4, 8, 1 << 31, null) == -2   # K > 2^31 - 1
    assert b"2^31-1" in lib.ggo_last_error()
    assert lib.gemm_ordered_grouped(null, 1, 0, null) == -1
    arr = (g.Problem * 1)()
    assert lib.gemm_ordered_grouped(arr, 17, 0, null) == -1
    # the grouped launch sizes its tile from the problems before it validates them: sizes that would overflow
    # that count, or negative ones, still end in an error code, with nothing launched
    big = (g.Problem * 2)()
    big[0].M, big[0].N, big[0].K, big[0].batch = 8, 1 << 40, 1 << 40, 1 << 40
    big[1].M, big[1].N, big[1].K, big[1].batch = 8, -5, 1 << 62, 3
    assert lib.gemm_ordered_grouped(big, 2, 0, null) < 0
    big[0].N, big[0].K, big[0].batch = -1, -1, -1
    assert lib.gemm_ordered_grouped(big, 1, 0, null) < 0
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
    """The handle API draws its signs from the seed (splitmix64, top bit): with the seed set to the key of
    the generator's stream they are the generator's signs, and every value and verdict equals the
    oracle's on the same signs."""
    x, W, r = synth.decode_gemv(2, 4, k=512, n=768)
    y = oracle.gemm_ordered(x, W)
    f = g.freivalds_prepare(W, synth.stream_key(2, "gemv.r"))
    assert np.array_equal(f.signs(), r)
    prep_a = g.freivalds_prepare_signs(W, r)
    prep_o = oracle.freivalds_prepare(W, r)
    for a, b in zip(prep_a, prep_o):
        assert np.array_equal(a, b)
    for m in range(4):
        yb = y[m].copy()
        if m == 3:
            yb[100] += np.float32(0.005)
        res_h = f.check(x[m], yb, 0.125)
        res_a = g.freivalds_check_signs(prep_a, r, x[m], yb, 0.125)
        res_o = oracle.freivalds_check(prep_o, r, x[m], yb, 0.125)
        assert res_h == res_a
        assert res_h[0] == res_o[0] == (m != 3)
        assert np.allclose(res_h[1:], res_o[1:], rtol=1e-12, atol=1e-15)
    f.close()
    f.close()   # a second close is a no-op


def test_freivalds_signs_follow_the_seed(g):
    """Sign n is the top bit of splitmix64 at counter n of the stream `seed`: the generator's definition,
    for several seeds, including 0 and the all-ones seed."""
    W = np.zeros((3, 1000), dtype=np.uint16)
    for seed in (0, 1, 12345, 2 ** 64 - 1, synth.stream_key(7, "x")):
        want = (1 - 2 * (synth.bits64(seed, 0, 1000) >> np.uint64(63)).astype(np.int64)).astype(np.int8)
        assert np.array_equal(g.freivalds_prepare(W, seed).signs(), want), seed
    # the two signs are about equally likely
    r = g.freivalds_prepare(np.zeros((1, 100000), dtype=np.uint16), 99).signs()
    assert abs(int(r.sum())) < 4 * 316


def test_freivalds_rejects_bad_arguments(g):
    W = np.zeros((4, 4), dtype=np.uint16)
    with pytest.raises(g.GGOError):
        g.freivalds_prepare_signs(W, np.array([1, 0, -1, 1], dtype=np.int8))
    lib = g.lib
    h = ct.c_void_p(1)
    assert lib.freivalds_prepare(None, 4, 4, 4, 0, ct.byref(h)) == -1 and h.value is None   # null W
    assert lib.freivalds_prepare(W.ctypes.data, 3, 4, 4, 0, ct.byref(h)) == -1             # ldw < N
    assert lib.freivalds_prepare(W.ctypes.data, 4, 4, 4, 0, None) == -1                     # null out
    out = np.empty(4)
    assert lib.freivalds_check(None, W.ctypes.data, W.ctypes.data, 0.125, out.ctypes.data) == -1
    lib.freivalds_free(None)


def test_gemv_instance_hook_rejects_what_it_cannot_run(g):
    lib, null = g.lib, None
    # unknown kind, bad rows, rows below M, bad form: all before any GPU call
    assert lib.ggo_test_gemv_instance(9, 1, 1, 16, 8, 16, 8, 16, 8, 1, 8, 8, null) == -1
    assert lib.ggo_test_gemv_instance(0, 3, 1, 16, 8, 16, 8, 16, 8, 1, 8, 8, null) == -1
    assert lib.ggo_test_gemv_instance(0, 2, 1, 16, 8, 16, 8, 16, 8, 4, 8, 8, null) == -2
    assert lib.ggo_test_gemv_instance(0, 4, 0, 16, 8, 16, 8, 16, 8, 4, 8, 8, null) == -1
    assert lib.ggo_test_gemv_instance(1, 4, 1, 16, 8, 16, 8, 16, 8, 4, 8, 8, null) == -1   # ordered takes rows 0
    assert lib.ggo_test_gemv_instance(3, 4, 1, 16, 8, 16, 8, 16, 8, 4, 8, 8, null) == -1   # mfma takes form 0
    # the persistent tree instance needs 16-byte operands, K <= 4096 and rows <= 8
    assert lib.ggo_test_gemv_instance(0, 16, 1, 16, 8, 16, 8, 16, 8, 4, 8, 8, null) == -2
    assert lib.ggo_test_gemv_instance(0, 4, 1, 16, 8200, 16, 8200, 16, 8, 4, 8, 8200, null) == -2
    assert lib.ggo_test_gemv_instance(0, 4, 1, 18, 8, 16, 8, 16, 8, 4, 8, 8, null) == -2
    # the 128-k ordered instance needs 4-byte column pairs of W
    assert lib.ggo_test_gemv_instance(1, 0, 2, 16, 8, 16, 7, 16, 8, 4, 7, 8, null) == -2
    assert lib.ggo_test_gemv_instance(1, 0, 2, 16, 8, 18, 8, 16, 8, 4, 8, 8, null) == -2
    # the 512-k ordered instance: W^T form only (form 3 of kind 2), M = 1, 16-byte operands
    assert lib.ggo_test_gemv_instance(1, 0, 3, 16, 8, 16, 8, 16, 8, 1, 8, 8, null) == -1
    assert lib.ggo_test_gemv_instance(2, 0, 3, 16, 8, 16, 8, 16, 8, 2, 8, 8, null) == -2
    assert lib.ggo_test_gemv_instance(2, 0, 3, 8, 8, 16, 8, 16, 8, 1, 8, 8, null) == -2
    assert lib.ggo_test_gemv_instance(2, 0, 5, 16, 8, 16, 8, 16, 8, 1, 8, 8, null) == -1
    # the MR-row ordered instance: W^T form only (form 4 of kind 2), rows 0, 2, 4 or 8, 16-byte operands
    assert lib.ggo_test_gemv_instance(1, 0, 4, 16, 8, 16, 8, 16, 8, 4, 8, 8, null) == -1
    assert lib.ggo_test_gemv_instance(2, 3, 4, 16, 8, 16, 8, 16, 8, 4, 8, 8, null) == -1
    assert lib.ggo_test_gemv_instance(2, 16, 4, 16, 8, 16, 8, 16, 8, 4, 8, 8, null) == -1
    assert lib.ggo_test_gemv_instance(2, 4, 4, 8, 8, 16, 8, 16, 8, 4, 8, 8, null) == -2   # x 8-byte aligned only
    assert lib.ggo_test_gemv_instance(2, 4, 4, 16, 12, 16, 12, 16, 8, 4, 8, 12, null) == -2   # K = 12
    # empty problems launch nothing
    assert lib.ggo_test_gemv_instance(0, 1, 2, null, 8, null, 8, null, 8, 0, 8, 8, null) == 0


def test_mfma_tile_hook_rejects_what_it_cannot_run(g):
    """ggo_test_gemm_mfma_tile: an unknown tile is refused, and the four direct-to-LDS tiles refuse
    operands they cannot load, all before any GPU call (fake addresses are never touched)."""
    lib, null = g.lib, None
    for tile in (-1, 6):
        assert lib.ggo_test_gemm_mfma_tile(tile, 16, 8, 16, 8, 16, 8, 4, 8, 8, null) == -1
    for tile in (0, 3, 4, 5):
        assert lib.ggo_test_gemm_mfma_tile(tile, 16, 12, 16, 8, 16, 8, 4, 8, 12, null) == -2   # K = 12
        assert lib.ggo_test_gemm_mfma_tile(tile, 18, 8, 16, 8, 16, 8, 4, 8, 8, null) == -2     # A misaligned
    # empty problems launch nothing, whatever the tile
    assert lib.ggo_test_gemm_mfma_tile(3, null, 8, null, 8, null, 8, 0, 8, 8, null) == 0
