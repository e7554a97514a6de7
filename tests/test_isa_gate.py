"""ISA gate over this repository's own gfx950 code objects.

The order contract forbids contraction ("Reproducible GPU inference": no fused
multiply-add, no fast-math), so the ordered kernels must hold no fused or dot
instruction and must hold separate binary32 multiplies and adds. The MFMA
kernel's order is fixed by its opcode ("Taming Bitwise Behavior in GPU Kernels
with Tensor Core", section 3.2.2: instruction_k), so it must use exactly one
matrix opcode. The tree-ordered GEMV folds each chain with one fused multiply-add
per k (section 3.2.2 of the same page, the scalar path's chain of fused
multiply-adds), so its floating-point arithmetic must be v_fma_f32 and plain
v_add_f32 only: no separate multiply, no packed, dot or matrix instruction.
No kernel may use atomics (arrival order would move bits).
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "gemv_gemm_ordered_amd", "_build")
LLVM = "/opt/rocm/llvm/bin"

# floating-point fused or dot forms (integer address arithmetic such as v_mad_u64_u32 is fine)
FUSED = re.compile(r"\b(v_(?:pk_)?(?:fma|fmac|mad|mac)_(?:f16|f32|f64|legacy\w*|mix\w*)|v_fma_mix\w*|v_dot\w*"
                   r"|v_pk_mul_f32|v_pk_add_f32)\b")
ATOMIC = re.compile(r"\b\w*atomic\w*\b")
MFMA = re.compile(r"\b(v_mfma\w*|v_smfmac\w*)\b")


def disassemble(obj):
    tmp = obj + ".fatbin"
    co = obj + ".gfx950.co"
    subprocess.run(["objcopy", "--dump-section", f".hip_fatbin={tmp}", obj], check=True)
    subprocess.run([f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o",
                    "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={tmp}", f"--output={co}"], check=True)
    out = subprocess.run([f"{LLVM}/llvm-objdump", "-d", "--no-show-raw-insn", co], check=True,
                         capture_output=True, text=True).stdout
    kernels, cur = {}, None
    for line in out.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\w+)>:", line)
        if m:
            cur = m.group(1)
            kernels[cur] = []
        elif cur and line.strip():
            kernels[cur].append(line.strip())
    return kernels


@pytest.fixture(scope="module")
def code():
    if not os.path.isdir(BUILD):
        pytest.skip("library not built")
    return {src: disassemble(os.path.join(BUILD, src + ".o"))
            for src in ("ordered_gemm.hip", "ordered_gemv.hip", "tree_gemv.hip", "mfma_invariant.hip", "mfma_gemv.hip",
                        "capi.cpp")}


def test_ordered_kernels_have_no_contraction(code):
    for src in ("ordered_gemm.hip", "ordered_gemv.hip"):
        ks = [k for k in code[src] if "ordered" in k]
        assert ks, src
        for k in ks:
            text = "\n".join(code[src][k])
            assert not FUSED.search(text), (k, FUSED.search(text).group(0))
            assert re.search(r"\bv_mul_f32", text) and re.search(r"\bv_add_f32", text), k
            assert not MFMA.search(text), k


def test_tree_kernels_use_single_fma_and_add(code):
    """The instances without an epilogue (template flag EPI = false, mangled ...Lb0EEEv8TreeArgs, or
    ...Lb0ELi<batch>ELb<contiguous>EEEv8TreeArgsi for the persistent form) hold
    the fold and the tree alone: their binary32 arithmetic is v_fma_f32 / v_fmac_f32 and v_add_f32 only.
    The epilogue instances add the epilogue's own operations after the fold; they are checked for no
    packed, dot or matrix instruction."""
    ks = [k for k in code["tree_gemv.hip"] if "k_gemv_tree" in k]
    # one-group form: M tiers 1, 2, 4, 8, 16 x 16-byte / 2-byte loads x with / without epilogue;
    # persistent form: M tiers 1, 2, 4, 8 x 1 or 2 steps per chain x with / without epilogue
    assert len([k for k in ks if "k_gemv_treeI" in k]) == 20, ks
    assert len([k for k in ks if "k_gemv_tree_pI" in k]) == 16, ks
    # the epilogue flag is the last bool template argument (the persistent form adds its batch size and its
    # group-mapping flag after it, and takes an int argument after TreeArgs)
    plain = [k for k in ks if k.endswith("Lb0EEEv8TreeArgs") or re.search(r"Lb0ELi\d+ELb[01]EEEv8TreeArgsi$", k)]
    assert len(plain) == 18, plain
    for k in ks:
        text = "\n".join(code["tree_gemv.hip"][k])
        assert not MFMA.search(text) and not re.search(r"\bv_dot|\bv_pk_(?:fma|mul|add)_f32", text), k
    float_op = re.compile(r"\bv_(?:pk_)?[a-z0-9]+_f(?:16|32|64)\w*")
    for k in plain:
        text = "\n".join(code["tree_gemv.hip"][k])
        ops = {m.group(0) for m in float_op.finditer(text)}
        ops = {o for o in ops if not o.startswith(("v_cvt", "v_cmp"))}
        assert ops <= {"v_fma_f32", "v_add_f32", "v_add_f32_e32", "v_add_f32_e64", "v_add_f32_dpp",
                       "v_fmac_f32", "v_fmac_f32_e32", "v_fmac_f32_e64"}, (k, ops)
        assert re.search(r"\bv_fmac?_f32", text), k
        assert not MFMA.search(text) and not re.search(r"\bv_dot", text), k


def test_mfma_kernels_use_one_opcode(code):
    """Every matrix-core kernel (both tile instances, both W layouts) issues one and the same
    opcode, so all of them fold each output with the same instruction_k."""
    ks = [k for k in code["mfma_invariant.hip"] if "k_gemm_mfma" in k]
    assert len(ks) >= 3, ks   # 256x128 (W and W^T) and the 128x128 instance
    for k in ks:
        ops = {m.group(1) for line in code["mfma_invariant.hip"][k] for m in [MFMA.search(line)] if m}
        assert ops == {"v_mfma_f32_16x16x32_bf16"}, (k, ops)
    # the matrix-core GEMV: staged x rows 1, 2, 4, 8, 16 x with / without the epilogue
    ks = [k for k in code["mfma_gemv.hip"] if "k_gemv_mfma" in k]
    assert len(ks) == 10, ks
    for k in ks:
        ops = {m.group(1) for line in code["mfma_gemv.hip"][k] for m in [MFMA.search(line)] if m}
        assert ops == {"v_mfma_f32_16x16x32_bf16"}, (k, ops)


def test_no_atomics_anywhere(code):
    for src, ks in code.items():
        for k, lines in ks.items():
            for line in lines:
                assert not ATOMIC.search(line), (src, k, line)


def test_hot_kernels_use_no_scratch(code):
    """The matrix-core, tree and ordered GEMV kernels keep all their state in registers and LDS. A scratch
    (private memory) access in them means an array the compiler could not keep in registers -- for
    example an accumulator array indexed with a runtime value -- and it turns every matrix
    instruction into a memory round trip while the results stay correct."""
    scratch = re.compile(r"\b(scratch_\w+|buffer_(?:load|store)_\w+ [^;]*\boff, s\[0:3\])")
    for src, tag in (("mfma_invariant.hip", "k_gemm_mfma"), ("tree_gemv.hip", "k_gemv_tree"),
                     ("mfma_gemv.hip", "k_gemv_mfma"), ("ordered_gemv.hip", "k_gemv_ordered")):
        ks = [k for k in code[src] if tag in k]
        assert ks, src
        for k in ks:
            hits = [line for line in code[src][k] if scratch.search(line)]
            assert not hits, (k, hits[:3])
