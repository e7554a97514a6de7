"""Pins for the oracle's tree-ordered GEMV (``oracle_gemv_tree``).

The order: "Taming Bitwise Behavior in GPU Kernels with Tensor Core", section 3.2.2 (GEMV paragraph,
Figure 2(d): the lanes take every countth tile of the k axis, each folds its tiles as a chain of fused
multiply-adds, and a butterfly combines the lanes) and section 5.1 (the pinned butterfly counts its
offsets up from 1, a balanced tree whose first level adds neighbours). This library fixes tiles of
8 k and 256 chains.

Each probe below places a few values on one row of x (every weight 1 unless stated) so that the
documented order gives one hand-derived value and each plausible mistake gives another:
  L = 1024, r = 2^-15 < half an ulp of L in binary32, so L + r rounds back to L.
The derivations are in the comments; none of the expected values comes from running the oracle.
The mutant gates at the end show that each pin fails when its part of the order is changed.
"""
import hashlib
import math
import os
import shutil

import numpy as np
import pytest

import oracle
import synth
from oracle import build as obuild
from tests.emulate import as_f64, bits, exact_dot, widen
from tests.test_oracle_pins import bf16_of

L = 1024.0
R = 2.0 ** -15
BF16_MAX = float.fromhex("0x1.fep+127")   # largest finite bfloat16, (2 - 2^-7) * 2^127


def probe(placed, K, weights=None):
    """x row with ``placed`` {k: value}, zeros elsewhere; W^T row of ones (or ``weights`` {k: value})."""
    xv = np.zeros(K, dtype=np.float32)
    for k, v in placed.items():
        xv[k] = v
    wv = np.ones(K, dtype=np.float32)
    for k, v in (weights or {}).items():
        wv[k] = v
    return bf16_of(xv)[None, :], bf16_of(wv)[None, :]


# name: (placed values, K, weights, expected value); the comments give the derivation and what a mistake gives
PROBES = {
    # chains 0, 2, 3 hold r, -L, L. Count-up tree: (c0 + c1) + (c2 + c3) = r + (-L + L) = r.
    # A left fold over k gives (r - L) + L = 0; a count-down (bit-reversed) tree pairs the even
    # chains first, (r + -L) = -L, then adds the odd total L: 0.
    "count_up_tree": ({0: R, 16: -L, 24: L}, 64, None, R),
    # k = 0, 2, 3 share tile 0, so one chain folds r, -L, L in order: (r - L) + L = 0.
    # Dealing single k instead of 8-k tiles puts them in chains 0, 2, 3: r (as above).
    "tile_of_8": ({0: R, 2: -L, 3: L}, 64, None, 0.0),
    # tiles 0 and 256 are both chain 0 (256 chains): chain 0 = -L + L = 0, chain 1 = r, total r.
    # With more than 256 chains tile 256 is its own chain: (-L + r) = -L meets L at the root: 0.
    "chains_not_more_than_256": ({0: -L, 8: R, 2048: L}, 2056, None, R),
    # tile 128 is chain 128 (256 chains): the left half of the tree totals -L + r = -L, the right
    # half L, total 0. With 128 chains tile 128 would join chain 0: (-L + L) + r = r.
    "chains_not_fewer_than_256": ({0: -L, 8: R, 1024: L}, 1032, None, 0.0),
    # tiles 0, 256, 512 of chain 0, ascending: (r - L) + L = 0. Descending: (L - L) + r = r.
    "chain_ascending": ({0: R, 2048: -L, 4096: L}, 4104, None, 0.0),
    # k = 0, 1, 2 inside tile 0, ascending: (r - L) + L = 0. Descending: (L - L) + r = r.
    "tile_ascending": ({0: R, 1: -L, 2: L}, 16, None, 0.0),
    # one fused rounding per step: fma(2^127, 3, -BF16_MAX) = 3 * 2^127 - (2^128 - 2^120)
    # = 2^127 + 2^120, finite. Rounding the product first overflows to +inf.
    "fused_multiply_add": ({0: -BF16_MAX, 1: 2.0 ** 127}, 8, {1: 3.0}, 2.0 ** 127 + 2.0 ** 120),
}


@pytest.mark.parametrize("name", sorted(PROBES))
def test_order_probe(name):
    placed, K, weights, want = PROBES[name]
    x, wt = probe(placed, K, weights)
    got = oracle.gemv_tree(x, wt)[0, 0]
    assert got == np.float32(want), (name, float(got), want)


def test_zero_is_positive_zero():
    # every product is -1 * 0 = -0; a chain started at +0 stays +0 (+0 + -0 = +0), and so does the tree
    x, wt = probe({k: -1.0 for k in range(40)}, 40, {k: 0.0 for k in range(40)})
    assert bits(oracle.gemv_tree(x, wt))[0, 0] == 0
    assert bits(oracle.gemv_tree(x[:, :0], wt[:, :0]))[0, 0] == 0      # K = 0: the empty sum is +0


def test_integer_data_exact_in_any_order():
    # integer products and sums below 2^24 are exact, so every order returns the exact dot product;
    # a dropped term, a wrong index or a transposed operand changes it
    x = synth.integer_bf16(1, "tree.x", (5, 3001))
    wt = synth.integer_bf16(1, "tree.wt", (37, 3001))
    y = oracle.gemv_tree(x, wt)
    exact = widen(x).astype(np.int64) @ widen(wt).astype(np.int64).T
    assert np.array_equal(y.astype(np.int64), exact)


@pytest.mark.parametrize("K", [1, 7, 8, 9, 100, 2048, 2049, 5000])
def test_within_the_tree_error_bound(K):
    # a chain of c fused steps and 8 tree levels: |y - exact| <= gamma_(c+8) * sum |x w|
    rng = np.random.default_rng(K)
    x = synth.f32_to_bf16_bits(rng.standard_normal((2, K)).astype(np.float32))
    wt = synth.f32_to_bf16_bits((rng.standard_normal((3, K)) * 0.02).astype(np.float32))
    y = oracle.gemv_tree(x, wt)
    a, w = as_f64(x), widen(wt).astype(np.float64)
    c = 8 * math.ceil(math.ceil(K / 8) / 256)
    u = 2.0 ** -24
    gamma = (c + 8) * u / (1 - (c + 8) * u)
    for m in range(2):
        for n in range(3):
            ex = float(exact_dot(a[m], w[n]))
            assert abs(ex - float(y[m, n])) <= gamma * float(np.abs(a[m] * w[n]).sum())


def test_rows_independent_of_M():
    x, W, _ = synth.decode_gemv(3, m_max=8, k=1000, n=64)
    wt = np.ascontiguousarray(W.T)
    full = bits(oracle.gemv_tree(x, wt))
    for M in range(1, 8):
        assert np.array_equal(bits(oracle.gemv_tree(x[:M], wt)), full[:M])
    assert np.array_equal(bits(oracle.gemv_tree(x, wt, threads=4)), full)


# ---- mutant gates: each planted change of the order must fail its pin ----

MUTANTS = {
    "count_down_tree": ("part[i] = part[2 * i] + part[2 * i + 1];", "part[i] = part[i] + part[i + width / 2];",
                        "count_up_tree"),
    "single_k_deal": ("#define TREE_TILE 8", "#define TREE_TILE 1", "tile_of_8"),
    "512_chains": ("#define TREE_CHAINS 256", "#define TREE_CHAINS 512", "chains_not_more_than_256"),
    "128_chains": ("#define TREE_CHAINS 256", "#define TREE_CHAINS 128", "chains_not_fewer_than_256"),
    "chain_descending": ("for (int64_t t = p; t * TREE_TILE < K; t += TREE_CHAINS) {",
                         "for (int64_t t = p + TREE_CHAINS * ((K / TREE_TILE - p) / TREE_CHAINS + 1); "
                         "(t -= TREE_CHAINS) >= p;) { if (t * TREE_TILE >= K) continue;",
                         "chain_ascending"),
    "tile_descending": ("for (int64_t k = k0; k < k1; ++k)", "for (int64_t k = k1 - 1; k >= k0; --k)",
                        "tile_ascending"),
    "separate_multiply": ("acc = fmaf(widen_bf16(xr[k]), widen_bf16(wr[k]), acc);",
                          "acc = acc + widen_bf16(xr[k]) * widen_bf16(wr[k]);", "fused_multiply_add"),
}


def build_mutant(tmp_path, name):
    old, new, _ = MUTANTS[name]
    tree = tmp_path / "oracle_copy"
    shutil.copytree(os.path.dirname(obuild.SRC), tree, ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    path = tree / "oracle.c"
    text = path.read_text()
    assert text.count(old) == 1, f"anchor for {name} not found exactly once"
    path.write_text(text.replace(old, new))
    lib = oracle.load(obuild.build(str(path), str(tree / "libmutant.so")))
    assert lib.oracle_source_sha256().decode() == hashlib.sha256(path.read_bytes()).hexdigest()
    return lib


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_its_pin(tmp_path, name):
    lib = build_mutant(tmp_path, name)
    placed, K, weights, want = PROBES[MUTANTS[name][2]]
    x, wt = probe(placed, K, weights)
    got = oracle.gemv_tree(x, wt, lib=lib)[0, 0]
    assert got != np.float32(want), f"mutant {name} still passes {MUTANTS[name][2]}"
    # and the mutant keeps integer data exact, so only the order pins can catch it
    xi = synth.integer_bf16(2, "tree.mx", (2, 700))
    wi = synth.integer_bf16(2, "tree.mw", (3, 700))
    assert np.array_equal(oracle.gemv_tree(xi, wi, lib=lib), oracle.gemv_tree(xi, wi))


def test_start_from_negative_zero_mutant(tmp_path):
    MUTANTS["neg_zero_start"] = ("float acc = 0.0f;\n                for (int64_t t = p;",
                                 "float acc = -0.0f;\n                for (int64_t t = p;", None)
    try:
        lib = build_mutant(tmp_path, "neg_zero_start")
    finally:
        del MUTANTS["neg_zero_start"]
    x, wt = probe({k: -1.0 for k in range(40)}, 40, {k: 0.0 for k in range(40)})
    assert bits(oracle.gemv_tree(x, wt, lib=lib))[0, 0] == 0x80000000
