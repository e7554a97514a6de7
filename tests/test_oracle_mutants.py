"""Mutant gates for the oracle: each planted fault must break a pin.

Method from "Same Bits on the CPU and the GPU" (section "A gate that read an
unmutated file"): one planted fault per gate, built from a copied tree, and a
build that can be shown to have read the mutated file. Here the copied source
is compiled by the same build function as the real oracle, and the library
reports the SHA-256 it was built from, which must be the mutant's.
"""
import hashlib
import os
import shutil

import numpy as np
import pytest

import oracle
import synth
from oracle import build as obuild
from tests.emulate import bits, fold_f64_emulated
from tests.test_oracle_pins import GOLD, bf16_of, hexf

FOLD_PROD = "const float p = a * widen_bf16(wrow[n]);   /* first rounding  */"
FOLD_ADD = "acc[n] = acc[n] + p;                        /* second rounding */"
K_LOOP = """        for (int64_t k = 0; k < K; ++k) {
            const float a = load_a(A, a_dtype, m * lda + k);"""

MUTANTS = {
    # ascending k becomes descending k
    "k_reversed": (K_LOOP, K_LOOP.replace("for (int64_t k = 0; k < K; ++k)", "for (int64_t k = K - 1; k >= 0; --k)")),
    # the last two k swap places (a swap of k=0 and k=1 would be invisible: the first add is exact)
    "k_swap_tail": (K_LOOP, K_LOOP.replace(
        "const float a = load_a(A, a_dtype, m * lda + k);",
        "const int64_t kk = (K >= 2 && k >= K - 2) ? (2 * K - 3 - k) : k;\n"
        "            const float a = load_a(A, a_dtype, m * lda + kk);\n"
        "            const uint16_t *wrow_ = W + kk * ldw;").replace("k < K; ++k) {", "k < K; ++k) {")),
    # multiply and add contracted into one fused rounding
    "fma": (FOLD_PROD + "\n                " + FOLD_ADD,
            "acc[n] = fmaf(a, widen_bf16(wrow[n]), acc[n]);"),
}


def build_mutant(tmp_path, name):
    src_dir = os.path.dirname(obuild.SRC)
    tree = tmp_path / "oracle_copy"
    shutil.copytree(src_dir, tree, ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    path = tree / "oracle.c"
    text = path.read_text()
    old, new = MUTANTS[name]
    assert text.count(old) == 1, f"anchor for {name} not found exactly once"
    text = text.replace(old, new)
    if name == "k_swap_tail":
        text = text.replace("const uint16_t *wrow = W + k * ldw;\n            for (int64_t n = 0; n < N; ++n) {\n                const float p",
                            "const uint16_t *wrow = wrow_;\n            for (int64_t n = 0; n < N; ++n) {\n                const float p", 1)
    path.write_text(text)
    lib_path = str(tree / "libmutant.so")
    obuild.build(str(path), lib_path)
    lib = oracle.load(lib_path)
    digest = hashlib.sha256(path.read_bytes()).hexdigest()
    assert lib.oracle_source_sha256().decode() == digest, "the mutant build did not read the mutated file"
    assert digest != obuild.sha256_file(obuild.SRC)
    return lib


def test_production_build_reports_its_source():
    assert oracle.load().oracle_source_sha256().decode() == obuild.sha256_file(obuild.SRC)


@pytest.mark.parametrize("name", ["k_reversed", "k_swap_tail"])
def test_k_order_mutants_break_parity(tmp_path, name):
    lib = build_mutant(tmp_path, name)
    A, W = synth.gpt2_projection(0, 16)
    good = bits(oracle.gemm_ordered(A, W))
    bad = bits(oracle.gemm_ordered(A, W, lib=lib))
    assert np.array_equal(good, bits(fold_f64_emulated(A, W)))
    frac = float((good != bad).mean())
    # reversing the whole chain moves most outputs; swapping only the last two adds changes an
    # output only where the two orders round differently, a small but nonzero share
    floor = 0.5 if name == "k_reversed" else 0.001
    assert frac > floor, f"{name}: only {frac:.3%} of outputs changed"
    if name == "k_reversed":
        g = GOLD["W1_order"]
        a = bf16_of([hexf(v) for v in g["a"]])[None, :]
        w = bf16_of([hexf(v) for v in g["w"]])[:, None]
        assert hex(bits(oracle.gemm_ordered(a, w, lib=lib))[0, 0]) == g["k_reversed_bits"]


def test_fma_mutant_breaks_parity_on_f32_A(tmp_path):
    lib = build_mutant(tmp_path, "fma")
    g = GOLD["W2_fma"]
    a = np.array([[hexf(v) for v in g["a"]]], dtype=np.float32)
    w = bf16_of([hexf(v) for v in g["w"]])[:, None]
    assert "0x%08x" % bits(oracle.gemm_ordered(a, w, lib=lib))[0, 0] == g["contracted_bits"]
    P, V = synth.pv_sequence(0, 0, 64, heads=1)
    good = bits(oracle.gemm_ordered(P[0], V[0]))
    bad = bits(oracle.gemm_ordered(P[0], V[0], lib=lib))
    assert (good != bad).mean() > 0.05


def test_fma_mutant_invisible_on_bf16_A(tmp_path):
    # bf16 x bf16 products have at most 16 significant bits and are exact in binary32, so an fma
    # returns the same bits as the separate pair: a gate on bf16 A alone could never fail.
    lib = build_mutant(tmp_path, "fma")
    A, W = synth.gpt2_projection(0, 16)
    assert np.array_equal(bits(oracle.gemm_ordered(A, W)), bits(oracle.gemm_ordered(A, W, lib=lib)))
