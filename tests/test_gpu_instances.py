"""Every kernel instance of the decode GEMVs gives the same bits at the same M.

The GEMV entry points pick an instance of their kernel from M (how many rows of x a workgroup stages;
for the ordered GEMV also 64- or 128-k stages, and for the tree GEMV the persistent or the one-group
form). "Taming Bitwise Behavior in GPU Kernels with Tensor Core", section 3.2.2: block sizes are speed
knobs that must not move an output's order. Here each instance is forced through the
ggo_test_gemv_instance hook on the same rows at the same M and compared bit for bit with the oracle
(and so with every other instance and with the entry point's own choice)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import dev_bf16, f32_bits, host_bits, say

pytestmark = pytest.mark.gpu

TIERS = (1, 2, 4, 8, 16)


@pytest.fixture(scope="module")
def g():
    import gemv_gemm_ordered_amd as g
    return g


@pytest.fixture(scope="module")
def decode():
    x, W, _ = synth.decode_gemv(3, m_max=16)
    WT = np.ascontiguousarray(W.T)
    say("instances: oracles at the decode shape 16x4096x4096")
    return {"x": x, "W": W, "WT": WT, "dx": dev_bf16(x), "dW": dev_bf16(W), "dWT": dev_bf16(WT),
            "tree": f32_bits(oracle.gemv_tree(x, WT, threads=16)),
            "ordered": f32_bits(oracle.gemm_ordered(x, W, threads=16))}


def tree_instances(M, K, wide):
    for rows in TIERS:
        if rows < M:
            continue
        yield rows, 2
        if wide and K <= 4096 and rows <= 8:
            yield rows, 1


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 9, 16])
def test_tree_instances_at_the_decode_shape(g, decode, M):
    entry = host_bits(g.gemv_tree(decode["dx"][:M], decode["dWT"]))
    assert np.array_equal(entry, decode["tree"][:M]), M
    for rows, form in tree_instances(M, 4096, True):
        say(f"gemv_tree instance rows={rows} form={form} M={M}")
        got = host_bits(g.test_gemv_instance("tree", rows, form, decode["dx"][:M], decode["dWT"]))
        assert np.array_equal(got, entry), (M, rows, form)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 9, 16])
def test_ordered_instances_at_the_decode_shape(g, decode, M):
    ref = decode["ordered"][:M]
    entry = host_bits(g.gemv_ordered_wt(decode["dx"][:M], decode["dWT"]))
    assert np.array_equal(entry, ref), M
    for kind, W in (("ordered", decode["dW"]), ("ordered_wt", decode["dWT"])):
        for form in (1, 2, 3) if kind == "ordered_wt" and M == 1 else (1, 2):
            say(f"gemv {kind} instance form={form} M={M}")
            got = host_bits(g.test_gemv_instance(kind, 0, form, decode["dx"][:M], W))
            assert np.array_equal(got, ref), (kind, M, form)
    assert np.array_equal(host_bits(g.gemv_ordered(decode["dx"][:M], decode["dW"])), ref), M
    for rows in (0, 2, 4, 8):   # the MR-row instance (W^T): any rows per workgroup at any M
        say(f"gemv ordered_wt instance form=4 rows={rows} M={M}")
        got = host_bits(g.test_gemv_instance("ordered_wt", rows, 4, decode["dx"][:M], decode["dWT"]))
        assert np.array_equal(got, ref), ("mr", M, rows)


@pytest.mark.parametrize("M", [1, 2, 4, 7, 16])
def test_mfma_gemv_instances_at_the_decode_shape(g, decode, M):
    entry = host_bits(g.gemv_mfma_invariant(decode["dx"][:M], decode["dWT"]))
    # the GEMM's bits on the same rows (its own tile, chosen without M)
    assert np.array_equal(entry, host_bits(g.gemm_mfma_invariant(decode["dx"][:M], decode["dW"]))), M
    for rows in TIERS:
        if rows < M:
            continue
        say(f"gemv_mfma instance rows={rows} M={M}")
        got = host_bits(g.test_gemv_instance("mfma", rows, 0, decode["dx"][:M], decode["dWT"]))
        assert np.array_equal(got, entry), (M, rows)


@pytest.mark.parametrize("M,N,K", [(1, 37, 200), (3, 100, 2056), (5, 33, 4096), (2, 300, 1000), (6, 17, 4104),
                                   (8, 129, 776), (1, 100, 4104), (1, 1000, 1536), (1, 17, 8), (3, 104, 1001),
                                   (7, 520, 777), (1, 8, 3), (16, 136, 600)])
def test_instances_on_ragged_shapes(g, M, N, K):
    x = synth.normal_bf16(M + N + K, "inst.x", (M, K))
    W = synth.normal_bf16(M + N + K, "inst.W", (K, N), 0.02)
    WT = np.ascontiguousarray(W.T)
    dx, dW, dWT = dev_bf16(x), dev_bf16(W), dev_bf16(WT)
    say(f"instances ragged M={M} N={N} K={K}")
    ref_t = f32_bits(oracle.gemv_tree(x, WT))
    for rows, form in tree_instances(M, K, K % 8 == 0):
        assert np.array_equal(host_bits(g.test_gemv_instance("tree", rows, form, dx, dWT)), ref_t), (rows, form)
    ref_o = f32_bits(oracle.gemm_ordered(x, W))
    for form in (1, 2):
        if form == 1 or (N % 2 == 0 and K % 4 == 0):   # the 128-k instance on W [K, N]: 4-byte column pairs
            assert np.array_equal(host_bits(g.test_gemv_instance("ordered", 0, form, dx, dW)), ref_o), form
        if K % 4 == 0:
            assert np.array_equal(host_bits(g.test_gemv_instance("ordered_wt", 0, form, dx, dWT)), ref_o), form
    if M == 1 and K % 8 == 0:   # the 512-k stages of the W^T form
        assert np.array_equal(host_bits(g.test_gemv_instance("ordered_wt", 0, 3, dx, dWT)), ref_o)
    if K % 8 == 0:   # the MR-row instance of the W^T form
        for rows in (2, 4, 8):
            assert np.array_equal(host_bits(g.test_gemv_instance("ordered_wt", rows, 4, dx, dWT)), ref_o), rows
    if K % 8 == 0:
        ref_m = f32_bits(oracle.gemm_mfma(x, W))
        for rows in TIERS:
            if rows >= M:
                assert np.array_equal(host_bits(g.test_gemv_instance("mfma", rows, 0, dx, dWT)), ref_m), rows


def test_narrow_operands_take_the_one_group_instances(g):
    """Misaligned views (2-byte loads): every one-group tree instance; the persistent one is refused."""
    xb = synth.normal_bf16(5, "inst.nx", (4, 1001))
    Wb = synth.normal_bf16(5, "inst.nW", (70, 1001), 0.02)
    dx, dW = dev_bf16(xb), dev_bf16(Wb)
    xv, Wv = dx[:, 1:1000], dW[:, 1:1000]
    ref = f32_bits(oracle.gemv_tree(np.ascontiguousarray(xb[:, 1:1000]), np.ascontiguousarray(Wb[:, 1:1000])))
    for rows in (4, 8, 16):
        assert np.array_equal(host_bits(g.test_gemv_instance("tree", rows, 2, xv, Wv)), ref), rows
    with pytest.raises(g.GGOError):
        g.test_gemv_instance("tree", 4, 1, xv, Wv)      # the persistent form needs 16-byte operands
