"""GPU parity of the matrix-core decode GEMV (gemv_mfma_invariant): bit for bit against the CPU bit
model of the matrix instruction (oracle.gemm_mfma) on the same seeded inputs, and against
gemm_mfma_invariant on the same operands (a decode step and a prefill agree); at the decode size in
full for every M from 1 to 16, on ragged and strided shapes, through the fused epilogue; operands it
cannot take are rejected."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import dev_bf16, dev_f32, f32_bits, host_bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import gemv_gemm_ordered_amd as g
    return g


@pytest.fixture(scope="module")
def decode():
    x, W, _ = synth.decode_gemv(0, m_max=16)
    WT = np.ascontiguousarray(W.T)
    say("gemv_mfma decode 16x4096x4096: bit model")
    ref = oracle.gemm_mfma(x, W, threads=16).view(np.uint32)
    return x, W, ref, dev_bf16(x), dev_bf16(W), dev_bf16(WT)


def test_decode_full_size_every_M(g, decode):
    x, W, ref, dx, dW, dWT = decode
    prefill = host_bits(g.gemm_mfma_invariant(dx, dW))
    assert np.array_equal(prefill, ref)
    for M in range(1, 17):
        say(f"gemv_mfma decode M={M}")
        got = host_bits(g.gemv_mfma_invariant(dx[:M], dWT))
        assert np.array_equal(got, ref[:M]), f"M={M}: {np.count_nonzero(got != ref[:M])} outputs differ"


def test_row_content_at_any_position(g, decode):
    x, W, ref, dx, dW, dWT = decode
    for M, pos in ((4, 0), (8, 5), (16, 15), (3, 2)):
        B = x[:M].copy()
        B[pos] = x[9]
        got = host_bits(g.gemv_mfma_invariant(dev_bf16(B), dWT))
        assert np.array_equal(got[pos], ref[9]), (M, pos)


@pytest.mark.parametrize("M,N,K", [
    (1, 1, 8), (1, 7, 32), (2, 9, 40), (3, 13, 512), (5, 100, 520), (8, 4095, 4096), (16, 33, 4104),
    (4, 17, 6144), (9, 5, 6152), (16, 3, 776), (7, 600, 16392), (6, 1376, 4096), (2, 11008, 512),
])
def test_ragged_shapes_equal_bit_model_and_gemm(g, M, N, K):
    x = synth.normal_bf16(M * 7 + N + K, "mgemv.x", (M, K))
    W = synth.normal_bf16(M * 7 + N + K, "mgemv.W", (K, N), 0.02)
    WT = np.ascontiguousarray(W.T)
    say(f"gemv_mfma ragged M={M} N={N} K={K}")
    ref = oracle.gemm_mfma(x, W, threads=8).view(np.uint32)
    got = host_bits(g.gemv_mfma_invariant(dev_bf16(x), dev_bf16(WT)))
    assert np.array_equal(got, ref)
    assert np.array_equal(host_bits(g.gemm_mfma_invariant(dev_bf16(x), dev_bf16(W))), ref)


def test_wide_exponent_range(g):
    """Products spread over many binades: the block alignment and truncation steps of the instruction
    model decide many bits here."""
    rng = np.random.default_rng(7)
    M, K, N = 6, 264, 72
    x = synth.f32_to_bf16_bits((rng.standard_normal((M, K)) * 2.0 ** rng.integers(-40, 40, (M, K))).astype(np.float32))
    W = synth.f32_to_bf16_bits((rng.standard_normal((K, N)) * 2.0 ** rng.integers(-60, 20, (K, N))).astype(np.float32))
    ref = oracle.gemm_mfma(x, W, threads=8).view(np.uint32)
    got = host_bits(g.gemv_mfma_invariant(dev_bf16(x), dev_bf16(np.ascontiguousarray(W.T))))
    assert np.array_equal(got, ref)


def test_strided_views(g):
    import torch
    M, N, K = 5, 40, 1032
    x = synth.normal_bf16(11, "mgemv.sx", (M, K))
    W = synth.normal_bf16(11, "mgemv.sW", (K, N), 0.02)
    ref = oracle.gemm_mfma(x, W, threads=8).view(np.uint32)
    xbig = torch.zeros((M, K + 24), dtype=torch.bfloat16, device="cuda")
    xbig[:, :K] = dev_bf16(x)
    wbig = torch.zeros((N, K + 8), dtype=torch.bfloat16, device="cuda")
    wbig[:, :K] = dev_bf16(np.ascontiguousarray(W.T))
    ybig = torch.full((M, N + 3), -7.0, device="cuda")
    g.gemv_mfma_invariant(xbig[:, :K], wbig[:, :K], y=ybig[:, :N])
    got = host_bits(ybig)
    assert np.array_equal(got[:, :N], ref)
    assert (got[:, N:] == np.float32(-7.0).view(np.uint32)).all(), "wrote outside y"


def test_empty_and_zero_K(g):
    import torch
    WT = torch.zeros((8, 0), dtype=torch.bfloat16, device="cuda")
    y = g.gemv_mfma_invariant(torch.zeros((3, 0), dtype=torch.bfloat16, device="cuda"), WT)
    assert (host_bits(y) == 0).all() and y.shape == (3, 8)
    y0 = g.gemv_mfma_invariant(torch.zeros((0, 16), dtype=torch.bfloat16, device="cuda"),
                               torch.zeros((8, 16), dtype=torch.bfloat16, device="cuda"))
    assert y0.shape == (0, 8)


@pytest.mark.parametrize("act,out", [("none", "f32"), ("silu", "bf16"), ("gelu_tanh", "f32"), ("relu", "bf16")])
def test_epilogue_equals_gemm_epilogue(g, act, out):
    M, N, K = 8, 264, 1024
    x = synth.normal_bf16(21, "mgemv.ex", (M, K))
    W = synth.normal_bf16(21, "mgemv.eW", (K, N), 0.02)
    bias = synth.normal_f32(21, "mgemv.eb", (N,))
    res = synth.normal_f32(21, "mgemv.er", (M, N))
    dx, dW, db, dr = dev_bf16(x), dev_bf16(W), dev_f32(bias), dev_f32(res)
    dWT = dev_bf16(np.ascontiguousarray(W.T))
    got = g.gemv_mfma_invariant_ep(dx, dWT, bias=db, act=act, residual=dr, out=out)
    want = g.gemm_mfma_invariant_ep(dx, dW, bias=db, act=act, residual=dr, out=out)
    import torch
    torch.cuda.synchronize()
    gb = got.view(torch.int16 if out == "bf16" else torch.int32).cpu().numpy()
    wb = want.view(torch.int16 if out == "bf16" else torch.int32).cpu().numpy()
    assert np.array_equal(gb, wb)
    ep = oracle.epilogue(oracle.gemm_mfma(x, W, threads=8), bias=bias, act=act, residual=res, out=out)
    assert np.array_equal(gb.view(np.uint16 if out == "bf16" else np.uint32),
                          np.asarray(ep).view(np.uint16 if out == "bf16" else np.uint32))


def test_rejects_what_it_cannot_take(g):
    import torch
    x = torch.zeros((2, 72), dtype=torch.bfloat16, device="cuda")
    WT = torch.zeros((16, 72), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(g.GGOError):
        g.gemv_mfma_invariant(x[:, :68], WT[:, :68])          # K % 8 != 0
    with pytest.raises(g.GGOError):
        g.gemv_mfma_invariant(x[:, 1:65], WT[:, :64])         # x not 16-byte aligned
    with pytest.raises(g.GGOError):
        g.gemv_mfma_invariant(torch.zeros((17, 64), dtype=torch.bfloat16, device="cuda"), WT[:, :64])   # M > 16
