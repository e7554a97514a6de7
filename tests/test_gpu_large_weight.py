"""Operands past 2^32 bytes: each GEMV and GEMM entry point on a 4.3 GB bfloat16 weight, and both GEMMs
on 4.3 GB of activation rows, sampled outputs bit for bit against the oracle.

At K = 4096 a row of W^T is 8 KiB, so rows 262144 and 524288 start at 2^31 and 2^32 bytes. The weight
repeats a seeded block of B = 4099 rows of W^T (or columns of W [K, N]) 128 times, N = 524672, and the
activations repeat a block of B rows of A the same way. B is odd, so it divides neither 2^18 nor 2^19:
an address that wrapped at 2^31 or 2^32 bytes would read another row of the block, and the sampled
outputs around those rows and at the end would move. Each sampled output needs only its own row of W^T
(column of W, row of A) and the other operand, so the oracle computes it on that row alone.
The kernels' row and stage bases are 64-bit and their in-range offsets 32-bit; these cases are the
largest operands the decode and prefill entry points are sized for here.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import dev_bf16, f32_bits, host_bits, say

pytestmark = pytest.mark.gpu

K = 4096
B = 4099
REPS = 128
N = B * REPS                                    # 524672 outputs, 4.30 GB of weight
ROW_BYTES = K * 2
SAMPLE = np.array([0, 1, (1 << 31) // ROW_BYTES - 1, (1 << 31) // ROW_BYTES, (1 << 31) // ROW_BYTES + 1,
                   (1 << 32) // ROW_BYTES - 1, (1 << 32) // ROW_BYTES, (1 << 32) // ROW_BYTES + 1, N - 2, N - 1])


@pytest.fixture(scope="module")
def g():
    import gemv_gemm_ordered_amd as g
    return g


@pytest.fixture(scope="module")
def block():
    """The seeded block (B rows of W^T), x with 8 rows, and the block rows behind the sampled outputs."""
    WT0 = synth.normal_bf16(21, "large.WT", (B, K), 0.02)
    x = synth.normal_bf16(21, "large.x", (8, K), 1.0)
    return WT0, x, np.ascontiguousarray(WT0[SAMPLE % B])


@pytest.fixture(scope="module")
def big_wt(block):
    import torch
    WT0, x, _ = block
    say(f"large weight: W^T [{N}, {K}] bf16, {N * ROW_BYTES / 1e9:.2f} GB")
    dWT = dev_bf16(WT0).repeat(REPS, 1)
    assert dWT.shape == (N, K) and dWT.is_contiguous()
    yield dWT, dev_bf16(x)
    del dWT
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def big_w(block):
    import torch
    WT0, x, _ = block
    say(f"large weight: W [{K}, {N}] bf16, {N * ROW_BYTES / 1e9:.2f} GB")
    dW = dev_bf16(np.ascontiguousarray(WT0.T)).repeat(1, REPS)
    assert dW.shape == (K, N) and dW.is_contiguous()
    yield dW, dev_bf16(x)
    del dW
    torch.cuda.empty_cache()


def sampled(y):
    """The sampled columns of a device output, as bits on the host."""
    return host_bits(y[:, SAMPLE.tolist()].contiguous())


def check(got, ref, name):
    bad = np.count_nonzero(got != ref)
    assert bad == 0, f"{name}: {bad} of {ref.size} sampled outputs differ from the oracle"


@pytest.mark.parametrize("M", [1, 8])
def test_tree_gemv(g, block, big_wt, M):
    _, x, rows = block
    dWT, dx = big_wt
    say(f"gemv_tree M={M} N={N} K={K}")
    check(sampled(g.gemv_tree(dx[:M], dWT)), f32_bits(oracle.gemv_tree(x[:M], rows)), f"gemv_tree M={M}")


def test_matrix_core_gemv(g, block, big_wt):
    _, x, rows = block
    dWT, dx = big_wt
    say(f"gemv_mfma_invariant M=4 N={N} K={K}")
    ref = oracle.gemm_mfma(x[:4], np.ascontiguousarray(rows.T)).view(np.uint32)
    check(sampled(g.gemv_mfma_invariant(dx[:4], dWT)), ref, "gemv_mfma_invariant M=4")


@pytest.mark.parametrize("M", [1, 4])
def test_ordered_gemv_wt(g, block, big_wt, M):
    _, x, rows = block
    dWT, dx = big_wt
    say(f"gemv_ordered_wt M={M} N={N} K={K}")
    ref = f32_bits(oracle.gemm_ordered(x[:M], np.ascontiguousarray(rows.T)))
    check(sampled(g.gemv_ordered_wt(dx[:M], dWT)), ref, f"gemv_ordered_wt M={M}")


@pytest.mark.parametrize("M", [1, 4])
def test_ordered_gemv_kn(g, block, big_w, M):
    _, x, rows = block
    dW, dx = big_w
    say(f"gemv_ordered (W [K, N]) M={M} N={N} K={K}")
    ref = f32_bits(oracle.gemm_ordered(x[:M], np.ascontiguousarray(rows.T)))
    check(sampled(g.gemv_ordered(dx[:M], dW)), ref, f"gemv_ordered M={M}")


def test_ordered_gemm(g, block, big_w):
    _, x, rows = block
    dW, dx = big_w
    say(f"gemm_ordered M=3 N={N} K={K}")
    ref = f32_bits(oracle.gemm_ordered(x[:3], np.ascontiguousarray(rows.T)))
    check(sampled(g.gemm_ordered(dx[:3], dW)), ref, "gemm_ordered M=3")


def test_matrix_core_gemm(g, block, big_w):
    _, x, rows = block
    dW, dx = big_w
    say(f"gemm_mfma_invariant M=3 N={N} K={K}")
    ref = oracle.gemm_mfma(x[:3], np.ascontiguousarray(rows.T)).view(np.uint32)
    check(sampled(g.gemm_mfma_invariant(dx[:3], dW)), ref, "gemm_mfma_invariant M=3")


@pytest.fixture(scope="module")
def big_a():
    """A [N, K] (the same 4.3 GB size, as rows of activations) repeating a seeded block of B rows, and a
    small weight W [K, 64]."""
    import torch
    A0 = synth.normal_bf16(22, "large.A", (B, K), 1.0)
    W = synth.normal_bf16(22, "large.W", (K, 64), 0.02)
    say(f"large activations: A [{N}, {K}] bf16, {N * ROW_BYTES / 1e9:.2f} GB")
    dA = dev_bf16(A0).repeat(REPS, 1)
    assert dA.shape == (N, K) and dA.is_contiguous()
    yield A0, W, dA, dev_bf16(W)
    del dA
    torch.cuda.empty_cache()


@pytest.mark.parametrize("entry", ["gemm_ordered", "gemm_mfma_invariant"])
def test_gemm_rows_past_2_32_bytes(g, big_a, entry):
    A0, W, dA, dW = big_a
    say(f"{entry} M={N} N=64 K={K}")
    got = host_bits(getattr(g, entry)(dA, dW)[SAMPLE.tolist()].contiguous())
    rows = np.ascontiguousarray(A0[SAMPLE % B])
    ref = f32_bits(oracle.gemm_ordered(rows, W)) if entry == "gemm_ordered" else oracle.gemm_mfma(rows, W).view(np.uint32)
    check(got, ref, entry)


def bf16_sampled(y):
    import torch
    torch.cuda.synchronize()
    return y[:, SAMPLE.tolist()].contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("entry", ["gemv_tree_ep", "gemm_mfma_invariant_ep"])
def test_fused_epilogue(g, block, big_wt, big_w, entry):
    """Bias, activation and residual indexed past 2^21 outputs, bfloat16 out, on the 4.3 GB weight."""
    _, x, rows = block
    M, act = (4, "silu") if entry == "gemv_tree_ep" else (3, "gelu_tanh")
    bias = synth.normal_f32(23, "large.bias", (N,), 0.1)
    res = synth.normal_f32(23, "large.res", (M, N), 1.0)
    from tests.gpu_util import dev_f32
    dbias, dres = dev_f32(bias), dev_f32(res)
    say(f"{entry} M={M} N={N} K={K} {act}, bias, residual, bf16 out")
    if entry == "gemv_tree_ep":
        y = g.gemv_tree_ep(big_wt[1][:M], big_wt[0], bias=dbias, act=act, residual=dres, out="bf16")
        Y = oracle.gemv_tree(x[:M], rows)
    else:
        y = g.gemm_mfma_invariant_ep(big_w[1][:M], big_w[0], bias=dbias, act=act, residual=dres, out="bf16")
        Y = oracle.gemm_mfma(x[:M], np.ascontiguousarray(rows.T))
    ref = oracle.epilogue(Y, bias=bias[SAMPLE], act=act, residual=np.ascontiguousarray(res[:, SAMPLE]), out="bf16")
    check(bf16_sampled(y), ref, entry)
