"""Mutant gates for the HIP library, on the CPU.

Method from "Same Bits on the CPU and the GPU" (section "A gate that read an unmutated file"): a planted
fault is built from a copied tree, and the build must be shown to have read the mutated file, or a
passing gate proves nothing. Each mutant here is one change of order in a kernel:

  ordered_k_reversed_in_8   the 16 x 16 ordered GEMM tile folds each run of 8 k in descending order
  mfma_group_swap           the matrix-core GEMM feeds the second 32-k group of each 64-k tile first

For each, the copied tree is compiled by the library's own build function; the test then shows that
  * the mutant library's ggo_build_info() names the mutated file's SHA-256 (and production's for the
    untouched files), so the build read the mutant;
  * the mutated kernels' gfx950 code differs from production's and the other kernels' does not, so the
    change reached the code object;
  * the same change of order planted in the oracle moves the bits of the workload the GPU parity gates
    compare (tests/test_gpu_ordered.py, tests/test_gpu_mfma.py), so those gates cannot pass on it.
The mutant kernels are never run: a planted mistake stays on the CPU, where it is planted in the oracle.
"""
import hashlib
import json
import os
import shutil

import numpy as np
import pytest

import oracle
import synth
from gemv_gemm_ordered_amd import build as gbuild
from oracle import build as obuild
from tests.emulate import bits
from tests.test_isa_gate import disassemble

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

HIP_MUTANTS = {
    "ordered_k_reversed_in_8": ("ordered_gemm.hip", [
        # each run of 8 k is read as two 16-byte halves of 4 k: take the halves in reverse and each half's
        # 4 k in reverse, so k runs 7, 6, ..., 0 within every run of 8
        ("const float4 a = av[c & 1][h], w = wv[c & 1][h];",
         "const float4 a0 = av[c & 1][1 - h], w0 = wv[c & 1][1 - h];\n"
         "                            const float4 a = make_float4(a0.w, a0.z, a0.y, a0.x), "
         "w = make_float4(w0.w, w0.z, w0.y, w0.x);"),
    ]),
    "mfma_group_swap": ("mfma_invariant.hip", [
        ("f.a[i] = *reinterpret_cast<const bf16x8*>(base + c.ra[g] + i * ROW16);",
         "f.a[i] = *reinterpret_cast<const bf16x8*>(base + c.ra[g ^ 1] + i * ROW16);"),
        ("const bf16x8 w = *reinterpret_cast<const bf16x8*>(base + c.rw[g] + (r - 1) * ROW16);",
         "const bf16x8 w = *reinterpret_cast<const bf16x8*>(base + c.rw[g ^ 1] + (r - 1) * ROW16);"),
        ("const char* w = base + c.rw[j] + g * 32 * G::CB * 16 + ((r - 1) & 1) * 4 * G::CB * 16;",
         "const char* w = base + c.rw[j] + (g ^ 1) * 32 * G::CB * 16 + ((r - 1) & 1) * 4 * G::CB * 16;"),
    ]),
}

# Kernels whose code each mutant must change (a fragment of the mangled name), and must leave alone.
CHANGED = {"ordered_k_reversed_in_8": "TileILi16ELi16ELi128E", "mfma_group_swap": "k_gemm_mfma_invariant"}


def build_hip_mutant(tmp_path, name):
    src, edits = HIP_MUTANTS[name]
    tree = tmp_path / "tree"
    csrc = tree / "gemv_gemm_ordered_amd" / "csrc"
    shutil.copytree(gbuild.CSRC, csrc)
    shutil.copytree(os.path.join(ROOT, "include"), tree / "include")
    path = csrc / src
    text = path.read_text()
    for old, new in edits:
        assert text.count(old) == 1, f"anchor for {name} not found exactly once: {old}"
        text = text.replace(old, new)
    path.write_text(text)
    lib = gbuild.build(csrc=str(csrc), lib=str(tree / "libggo_mutant.so"), build_dir=str(tree / "_build"),
                       only=[src])
    return path, lib, tree / "_build" / (src + ".o")


def kernels_of(obj):
    """Each kernel's instructions without the disassembler's comments (they hold absolute addresses, which
    move when an earlier kernel in the object changes size)."""
    return {k: [ln.split("//")[0].strip() for ln in v] for k, v in disassemble(str(obj)).items()}


@pytest.fixture(scope="module")
def production_code():
    if not os.path.isdir(gbuild.BUILD_DIR):
        pytest.skip("library not built")
    return {s: kernels_of(os.path.join(gbuild.BUILD_DIR, s + ".o")) for s in ("ordered_gemm.hip", "mfma_invariant.hip")}


@pytest.mark.parametrize("name", sorted(HIP_MUTANTS))
def test_mutant_build_reads_the_mutated_file_and_changes_the_kernel(tmp_path, production_code, name):
    import ctypes as ct
    src = HIP_MUTANTS[name][0]
    path, lib_path, obj = build_hip_mutant(tmp_path, name)
    lib = ct.CDLL(lib_path)
    lib.ggo_build_info.restype = ct.c_char_p
    info = json.loads(lib.ggo_build_info().decode())
    digest = hashlib.sha256(path.read_bytes()).hexdigest()
    assert info["sources"][src] == digest, "the mutant build did not read the mutated file"
    assert digest != gbuild._sha(os.path.join(gbuild.CSRC, src))
    for other in gbuild.SOURCES:
        if other != src:
            assert info["sources"][other] == gbuild._sha(os.path.join(gbuild.CSRC, other)), other
    prod, mut = production_code[src], kernels_of(obj)
    assert set(prod) == set(mut)
    changed = {k for k in prod if prod[k] != mut[k]}
    assert changed, "the mutation did not reach the code object"
    assert all(CHANGED[name] in k for k in changed), sorted(changed)
    assert any(CHANGED[name] in k for k in prod)


ORACLE_FOLD = """const float a = load_a(A, a_dtype, m * lda + k);
            const uint16_t *wrow = W + k * ldw;"""
ORACLE_MFMA = """            for (int64_t k0 = 0; k0 < K; k0 += 8) {
                const int len = (int)(K - k0 < 8 ? K - k0 : 8);"""

ORACLE_MUTANTS = {
    # each aligned run of 8 k in descending order (k xor 7), as the ordered mutant folds it
    "ordered_k_reversed_in_8": [(ORACLE_FOLD, "const int64_t kx = ((k | 7) < K) ? (k ^ 7) : k;\n"
                                              "            const float a = load_a(A, a_dtype, m * lda + kx);\n"
                                              "            const uint16_t *wrow = W + kx * ldw;")],
    # the two 32-k groups of every 64-k tile swapped (k xor 32 on the blocks of 8), as the MFMA mutant feeds them
    "mfma_group_swap": [(ORACLE_MFMA, """            for (int64_t kb = 0; kb < K; kb += 8) {
                const int64_t k0 = (kb ^ 32) < K ? (kb ^ 32) : kb;
                const int len = (int)(K - k0 < 8 ? K - k0 : 8);""")],
}


def build_oracle_mutant(tmp_path, name):
    tree = tmp_path / "oracle_copy"
    shutil.copytree(os.path.dirname(obuild.SRC), tree, ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    path = tree / "oracle.c"
    text = path.read_text()
    for old, new in ORACLE_MUTANTS[name]:
        assert text.count(old) == 1, f"anchor for {name} not found exactly once: {old}"
        text = text.replace(old, new)
    path.write_text(text)
    lib = oracle.load(obuild.build(str(path), str(tree / "libmutant.so")))
    assert lib.oracle_source_sha256().decode() == hashlib.sha256(path.read_bytes()).hexdigest()
    return lib


def test_the_ordered_mutants_order_breaks_the_gpt2_gate(tmp_path):
    """The GPT-2 projection (K = 768: six whole 128-k steps of the 16 x 16 tile, so the GPU mutant folds
    exactly k xor 7) is compared with the oracle bit for bit on the GPU; under the mutant's order most of
    its outputs move."""
    lib = build_oracle_mutant(tmp_path, "ordered_k_reversed_in_8")
    A, W = synth.gpt2_projection(0, 16)
    good, bad = bits(oracle.gemm_ordered(A, W)), bits(oracle.gemm_ordered(A, W, lib=lib))
    assert (good != bad).mean() > 0.3


def test_the_mfma_mutants_order_breaks_the_bit_model_gate(tmp_path):
    """The matrix-core GEMM is compared with the bit model on the GPT-2 shape (K = 768, twelve whole 64-k
    tiles); with the groups of each tile swapped the model's bits move."""
    lib = build_oracle_mutant(tmp_path, "mfma_group_swap")
    A, W = synth.gpt2_projection(0, 8)
    good, bad = bits(oracle.gemm_mfma(A, W)), bits(oracle.gemm_mfma(A, W, lib=lib))
    assert (good != bad).mean() > 0.1
    # and on integer data every order is exact: the mutant is invisible there (why the model gate uses
    # real-valued data)
    Ai, Wi = synth.integer_bf16(1, "mut.Ai", (4, 256)), synth.integer_bf16(1, "mut.Wi", (256, 16))
    assert np.array_equal(bits(oracle.gemm_mfma(Ai, Wi)), bits(oracle.gemm_mfma(Ai, Wi, lib=lib)))
