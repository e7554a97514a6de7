"""GPU tests of the matrix-core path: bitwise batch invariance across M and row
position, the error bound against the binary64 reference, and the integer case
where every summation order is exact (so the output must equal the oracle
bit for bit)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import dev_bf16, f32_bits, host_bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import gemv_gemm_ordered_amd as g
    return g


def assert_within_bound(C, A, W, rows=None):
    """|c - c*| <= 2 K 2^-24 sum|a w| + 2^-8 |c*| for every checked element."""
    if rows is not None:
        A = np.ascontiguousarray(A[rows])
        C = C[rows]
    D = oracle.gemm_f64(A, W, threads=16)
    S = oracle.gemm_absdot_f64(A, W, threads=16)
    K = A.shape[1]
    bound = 2.0 * K * 2.0 ** -24 * S + 2.0 ** -8 * np.abs(D)
    err = np.abs(C.astype(np.float64) - D)
    assert (err <= bound).all(), f"max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3g}"
    return float(np.max(err / np.maximum(bound, 1e-300)))


def test_integer_data_exact(g):
    for (M, N, K) in [(200, 300, 1000), (1, 1, 1), (129, 130, 4096), (64, 128, 32), (7, 33, 65)]:
        A = synth.integer_bf16(M, "mi.A", (M, K))
        W = synth.integer_bf16(N, "mi.W", (K, N))
        ref = f32_bits(oracle.gemm_ordered(A, W, threads=16))
        got = host_bits(g.gemm_mfma_invariant(dev_bf16(A), dev_bf16(W)))
        assert np.array_equal(got, ref), (M, N, K)


def test_gpt2_rows_identical_for_every_M_1_to_512(g):
    A, W = synth.gpt2_projection(0, 512)
    dA, dW = dev_bf16(A), dev_bf16(W)
    full = host_bits(g.gemm_mfma_invariant(dA, dW))
    assert_within_bound(full.view(np.float32), A, W)
    say("mfma gpt2 M=1..512")
    for M in range(1, 513):
        got = host_bits(g.gemm_mfma_invariant(dA[:M], dW))
        assert np.array_equal(got, full[:M]), M


def test_mlp_sweep_invariant_and_bounded(g):
    A, W = synth.mlp_up(0, 2048)
    dA, dW = dev_bf16(A), dev_bf16(W)
    full = host_bits(g.gemm_mfma_invariant(dA, dW))
    for M in (64, 128, 256, 512, 1024):
        assert np.array_equal(host_bits(g.gemm_mfma_invariant(dA[:M], dW)), full[:M]), M
    rows = np.arange(0, 2048, 7)
    r = assert_within_bound(full.view(np.float32), A, W, rows)
    say(f"mlp max err/bound {r:.3g}")


def test_row_position_and_repeat(g):
    A, W = synth.mlp_up(1, 300)
    dW = dev_bf16(W)
    base = host_bits(g.gemm_mfma_invariant(dev_bf16(A), dW))
    for pos in (0, 127, 128, 255, 299):
        B = A.copy()
        B[pos] = A[17]
        assert np.array_equal(host_bits(g.gemm_mfma_invariant(dev_bf16(B), dW))[pos], base[17])
    for _ in range(3):
        assert np.array_equal(host_bits(g.gemm_mfma_invariant(dev_bf16(A), dW)), base)


@pytest.mark.parametrize("M,N,K", [(37, 333, 129), (130, 70, 33), (1, 1000, 4095), (256, 129, 31)])
def test_ragged_bounded_and_invariant(g, M, N, K):
    A = synth.normal_bf16(M, "mr.A", (M, K))
    W = synth.normal_bf16(N, "mr.W", (K, N), 0.02)
    dA, dW = dev_bf16(A), dev_bf16(W)
    C = host_bits(g.gemm_mfma_invariant(dA, dW))
    assert_within_bound(C.view(np.float32), A, W)
    # each single row alone gives the same bits
    for m in (0, M - 1):
        assert np.array_equal(host_bits(g.gemm_mfma_invariant(dA[m:m + 1], dW))[0], C[m])
    # misaligned / strided views give the same bits
    dAp = dev_bf16(np.pad(A, ((0, 0), (1, 0))))
    assert np.array_equal(host_bits(g.gemm_mfma_invariant(dAp[:, 1:], dW)), C)


@pytest.mark.parametrize("n", [4096, 11008])
def test_7b_projection_sampled(g, n):
    say(f"mfma 7b n={n}")
    A, W = synth.proj_7b(0, n)
    dA, dW = dev_bf16(A), dev_bf16(W)
    full = host_bits(g.gemm_mfma_invariant(dA, dW))
    rows = np.array([0, 1, 1000, 2047, 4095])
    assert_within_bound(full.view(np.float32), A, W, rows)
    sub = host_bits(g.gemm_mfma_invariant(dA[1000:1128], dW))
    assert np.array_equal(sub, full[1000:1128])


TILES = ("256x128", "256x256", "128x128_lds", "64x128_lds", "128x128", "64x64")
WIDE = ("256x128", "256x256", "128x128_lds", "64x128_lds")   # need K and N multiples of 8 (and aligned operands)


@pytest.mark.parametrize("M,N,K", [(256, 128, 64), (300, 200, 100), (513, 1000, 1111), (1, 4096, 4096),
                                   (2048, 4096, 1024), (4096, 4096, 4096), (4096, 11008, 4096), (7, 33, 31),
                                   (513, 1000, 1112), (300, 200, 104), (257, 136, 1000), (1, 8, 8), (255, 1032, 72)])
def test_tile_instances_agree_bitwise(g, M, N, K):
    """The six tile instances (four direct-to-LDS, two register-staged) feed every output the same operand values in the
    same 32-k groups ("Taming Bitwise Behavior in GPU Kernels with Tensor Core", section 3.2.2: block
    sizes do not enter the order), so their outputs, and the entry point's, must be identical bit for bit."""
    say(f"mfma tile instances M={M} N={N} K={K}")
    A = synth.normal_bf16(M + 1, "ti.A", (M, K))
    W = synth.normal_bf16(N + 2, "ti.W", (K, N), 0.02)
    dA, dW = dev_bf16(A), dev_bf16(W)
    entry = host_bits(g.gemm_mfma_invariant(dA, dW))
    for tile in TILES:
        if tile in WIDE and (K % 8 or N % 8):
            continue
        got = host_bits(g.test_gemm_mfma_tile(tile, dA, dW))
        assert np.array_equal(got, entry), f"{tile}: {np.count_nonzero(got != entry)} outputs differ"
    assert np.array_equal(host_bits(g.test_gemm_mfma_tile128(dA, dW)), entry)


@pytest.mark.parametrize("M,N,K", [(256, 128, 64), (300, 200, 104), (513, 1000, 1112), (1, 4096, 4096),
                                   (2048, 4096, 1024), (4096, 11008, 4096), (7, 40, 32), (130, 137, 1000)])
def test_transposed_w_entry_gives_the_same_bits(g, M, N, K):
    """gemm_mfma_invariant_wt(A, W^T) feeds every MFMA the same operand values as
    gemm_mfma_invariant(A, W), so the outputs must agree bit for bit."""
    import torch
    say(f"mfma W^T M={M} N={N} K={K}")
    A = synth.normal_bf16(M + 3, "wt.A", (M, K))
    W = synth.normal_bf16(N + 4, "wt.W", (K, N), 0.02)
    dA, dW = dev_bf16(A), dev_bf16(W)
    ref = host_bits(g.gemm_mfma_invariant(dA, dW))
    # the W^T entry wants row strides that are multiples of 8: hold A and W^T in padded buffers
    ld = (K + 7) // 8 * 8

    def padded(x, rows, extra=0):
        buf = torch.zeros((rows, ld + extra), dtype=torch.bfloat16, device="cuda")
        buf[:, :K] = x
        return buf[:, :K]

    Ap, WTp = padded(dA, M), padded(dW.t(), N)
    assert np.array_equal(host_bits(g.gemm_mfma_invariant_wt(Ap, WTp)), ref)
    # a wider W^T row stride (still a multiple of 8)
    assert np.array_equal(host_bits(g.gemm_mfma_invariant_wt(Ap, padded(dW.t(), N, 8))), ref)


def test_transposed_w_entry_rejects_misaligned(g):
    import torch
    A = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    WT = torch.zeros((8, 65), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(g.GGOError, match="aligned"):
        g.gemm_mfma_invariant_wt(A, WT[:, 1:])
    A2 = torch.zeros((4, 16), dtype=torch.bfloat16, device="cuda")[:, :12]   # K = 12: not a multiple of 8
    WT2 = torch.zeros((8, 16), dtype=torch.bfloat16, device="cuda")[:, :12]
    with pytest.raises(g.GGOError, match="multiple of 8"):
        g.gemm_mfma_invariant_wt(A2, WT2)


# ---- bit for bit against the CPU bit model of the matrix instruction (oracle.gemm_mfma) ----

def _wt(dW):
    return dW.t().contiguous()


def test_gpt2_bits_equal_cpu_model(g):
    A, W = synth.gpt2_projection(0, 512)
    say("mfma gpt2 512x768x768 vs bit model")
    ref = oracle.gemm_mfma(A, W, threads=16).view(np.uint32)
    dA, dW = dev_bf16(A), dev_bf16(W)
    for name, C in [("entry", g.gemm_mfma_invariant(dA, dW)), ("W^T", g.gemm_mfma_invariant_wt(dA, _wt(dW)))] + \
            [(t, g.test_gemm_mfma_tile(t, dA, dW)) for t in TILES]:
        got = host_bits(C)
        assert np.array_equal(got, ref), f"{name}: {np.count_nonzero(got != ref)} outputs differ from the model"
    for M in (1, 7, 64, 257):
        assert np.array_equal(host_bits(g.gemm_mfma_invariant(dA[:M], dW)), ref[:M]), M


@pytest.mark.parametrize("M,N,K", [(37, 333, 129), (130, 70, 33), (1, 1000, 4095), (256, 129, 31),
                                   (300, 200, 1000), (513, 1000, 1112), (5, 64, 8)])
def test_ragged_bits_equal_cpu_model(g, M, N, K):
    A = synth.normal_bf16(M + N + K, "mfma.bits.A", (M, K))
    W = synth.normal_bf16(M + N + K, "mfma.bits.W", (K, N), 0.02)
    say(f"mfma ragged {M}x{N}x{K} vs bit model")
    ref = oracle.gemm_mfma(A, W, threads=16).view(np.uint32)
    dA, dW = dev_bf16(A), dev_bf16(W)
    assert np.array_equal(host_bits(g.gemm_mfma_invariant(dA, dW)), ref)
    for tile in TILES:
        if tile not in WIDE or (K % 8 == 0 and N % 8 == 0):
            assert np.array_equal(host_bits(g.test_gemm_mfma_tile(tile, dA, dW)), ref), tile
    if K % 8 == 0:
        assert np.array_equal(host_bits(g.gemm_mfma_invariant_wt(dA, _wt(dW))), ref)


def test_wide_exponent_range_bits_equal_cpu_model(g):
    # operands over 2^-60 .. 2^60 and subnormal products: the alignment, truncation and subnormal steps
    rng = np.random.default_rng(9)
    A = synth.f32_to_bf16_bits((rng.standard_normal((64, 256)) * 2.0 ** rng.integers(-60, 60, (64, 256))).astype(np.float32))
    W = synth.f32_to_bf16_bits((rng.standard_normal((256, 96)) * 2.0 ** rng.integers(-60, 20, (256, 96))).astype(np.float32))
    ref = oracle.gemm_mfma(A, W, threads=16).view(np.uint32)
    assert np.array_equal(host_bits(g.gemm_mfma_invariant(dev_bf16(A), dev_bf16(W))), ref)


@pytest.mark.parametrize("name,M,n", [("mlp_up", 2048, 4096), ("7b", 4096, 4096), ("7b", 4096, 11008)])
def test_full_size_sampled_rows_equal_cpu_model(g, name, M, n):
    if name == "mlp_up":
        A, W = synth.mlp_up(0, M)
    else:
        A, W = synth.proj_7b(0, n=n, m=M)
    rows = np.array([0, 1, M // 2, M - 1])
    say(f"mfma {name} {M}x{n} sampled rows vs bit model")
    ref = oracle.gemm_mfma(A[rows], W, threads=16).view(np.uint32)
    dA, dW = dev_bf16(A), dev_bf16(W)
    got = host_bits(g.gemm_mfma_invariant(dA, dW))[rows]
    assert np.array_equal(got, ref)
    got_wt = host_bits(g.gemm_mfma_invariant_wt(dA, _wt(dW)))[rows]
    assert np.array_equal(got_wt, ref)


def test_hipblaslt_control_rows_move_with_M(g):
    """The control of the invariance tests: the vendor GEMM (hipBLASLt through torch.mm, binary32 out)
    on the same data gives row 0 different bits at some M, while gemm_mfma_invariant gives the same
    bits at every M. Without the control the invariance checks would not show anything."""
    import torch
    A = dev_bf16(synth.normal_bf16(41, "ctl.A", (2048, 1024)))
    W = dev_bf16(synth.normal_bf16(41, "ctl.W", (1024, 4096), 0.02))
    say("hipBLASLt control, MLP shape")
    ref_m = g.gemm_mfma_invariant(A, W)[0].view(torch.int32).clone()
    ref_b = torch.mm(A, W, out_dtype=torch.float32)[0].view(torch.int32).clone()
    moved_b = []
    for M in (1, 2, 8, 64, 128, 256, 512, 1024):
        assert torch.equal(g.gemm_mfma_invariant(A[:M], W)[0].view(torch.int32), ref_m), M
        if not torch.equal(torch.mm(A[:M], W, out_dtype=torch.float32)[0].view(torch.int32), ref_b):
            moved_b.append(M)
    assert moved_b, "hipBLASLt gave row 0 the same bits at every M: the control shows nothing here"
