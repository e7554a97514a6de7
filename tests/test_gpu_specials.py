"""IEEE special values inside the operands: infinities, NaN, products that overflow binary32, Inf x 0 and
Inf - Inf, through every GEMV and GEMM entry point, against the oracle on the same inputs.

Every step of the ordered and tree orders is one binary32 operation (a product, a sum or a fused
multiply-add), so where an output is not NaN its bits must equal the oracle's, and an output must be NaN
exactly where the oracle's is. A NaN's sign and payload are not compared: IEEE 754 leaves them open, and
the host and the GPU produce different default NaNs.

The oracle's bit model of the matrix instruction covers finite operands only (it reads an exponent field
of all ones as a number). For the matrix-core path, outputs whose row of x and column of W hold no special
value are compared bit for bit with that model. The others must match the ordered oracle's class: NaN,
+Inf or -Inf. IEEE arithmetic fixes that class whatever the order of the sum, as long as no finite partial
sum overflows, which these operands (no overflowing products) rule out.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import dev_bf16, f32_bits, host_bits, say

pytestmark = pytest.mark.gpu

M, N, K = 3, 200, 1000
PINF, NINF, QNAN = np.uint16(0x7F80), np.uint16(0xFF80), np.uint16(0x7FC0)


def bf16(v):
    return synth.f32_to_bf16_bits(np.array([v], dtype=np.float32))[0]


@pytest.fixture(scope="module")
def g():
    import gemv_gemm_ordered_amd as g
    return g


def operands(overflow):
    """x [M, K] and W^T [N, K] (bf16 bits) with specials planted at fixed places."""
    x = synth.normal_bf16(31, "specials.x", (M, K), 1.0).copy()
    WT = synth.normal_bf16(31, "specials.WT", (N, K), 0.02).copy()
    x[0, 5] = PINF                     # row 0: +-Inf times every w[n, 5]
    WT[7, 9] = QNAN                    # column 7: NaN in every row
    x[2, 30] = NINF
    WT[13, 30] = 0                     # (2, 13): -Inf x 0 = NaN
    x[1, 40] = x[1, 41] = bf16(1.0)
    WT[17, 40], WT[17, 41] = PINF, NINF     # column 17: +Inf - Inf = NaN in rows 1 and 2 at least
    WT[19, 50] = NINF                  # column 19: -Inf x x[m, 50]
    if overflow:
        x[1, 60] = bf16(3.0e38)
        WT[11, 60] = bf16(100.0)       # (1, 11): the product overflows to +Inf
        WT[23, 60] = bf16(-100.0)      # (1, 23): to -Inf
    return x, WT


def same(got, ref, name):
    """Bits equal where the reference is not NaN, and NaN in the same places."""
    gf, rf = got.view(np.float32), ref.view(np.float32)
    gn, rn = np.isnan(gf), np.isnan(rf)
    assert np.array_equal(gn, rn), f"{name}: NaN at {np.argwhere(gn != rn)[:8].tolist()} differs from the oracle"
    bad = (got != ref) & ~rn
    assert not bad.any(), f"{name}: {int(bad.sum())} non-NaN outputs differ, first at {np.argwhere(bad)[0].tolist()}"
    assert rn.any() and np.isinf(rf).any(), "the planted specials must reach the outputs"


@pytest.mark.parametrize("entry", ["gemm_ordered", "gemv_ordered", "gemv_ordered_wt"])
def test_ordered(g, entry):
    x, WT = operands(overflow=True)
    W = np.ascontiguousarray(WT.T)
    ref = f32_bits(oracle.gemm_ordered(x, W))
    assert np.isposinf(ref.view(np.float32)[1, 11]) and np.isneginf(ref.view(np.float32)[1, 23])
    say(f"specials: {entry} {M}x{N}x{K}")
    dx = dev_bf16(x)
    got = getattr(g, entry)(dx, dev_bf16(WT) if entry == "gemv_ordered_wt" else dev_bf16(W))
    same(host_bits(got), ref, entry)


@pytest.mark.parametrize("rows", [1, M])
def test_tree(g, rows):
    x, WT = operands(overflow=True)
    ref = f32_bits(oracle.gemv_tree(x[:rows], WT))
    say(f"specials: gemv_tree {rows}x{N}x{K}")
    same(host_bits(g.gemv_tree(dev_bf16(x[:rows]), dev_bf16(WT))), ref, f"gemv_tree M={rows}")


@pytest.mark.parametrize("entry", ["gemm_mfma_invariant", "gemv_mfma_invariant"])
def test_matrix_core(g, entry):
    x, WT = operands(overflow=False)
    W = np.ascontiguousarray(WT.T)
    special = lambda a: (a & 0x7F80) == 0x7F80
    touched = special(x).any(axis=1)[:, None] | special(WT).any(axis=1)[None, :]
    model = oracle.gemm_mfma(x, W).view(np.uint32)
    ordered = oracle.gemm_ordered(x, W)
    say(f"specials: {entry} {M}x{N}x{K}")
    got = host_bits(getattr(g, entry)(dev_bf16(x), dev_bf16(W) if entry == "gemm_mfma_invariant" else dev_bf16(WT)))
    bad = (got != model) & ~touched
    assert not bad.any(), f"{entry}: {int(bad.sum())} outputs without specials differ from the bit model"
    gf = got.view(np.float32)
    for cls in (np.isnan, np.isposinf, np.isneginf):
        mism = (cls(gf) != cls(ordered)) & touched
        assert not mism.any(), f"{entry}: {cls.__name__} differs at {np.argwhere(mism)[:8].tolist()}"
    assert touched.any() and (~touched).any()
