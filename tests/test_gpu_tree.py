"""GPU parity of the tree-ordered GEMV (gemv_tree): bit for bit against the CPU oracle on the same
seeded inputs, at the decode size in full and on ragged, strided and misaligned shapes; bits
independent of M; the order probes of the oracle's pins give the same hand-derived values."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import dev_bf16, f32_bits, host_bits, say
from tests.test_oracle_tree import PROBES, probe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import gemv_gemm_ordered_amd as g
    return g


@pytest.fixture(scope="module")
def decode():
    x, W, _ = synth.decode_gemv(0, m_max=16)
    WT = np.ascontiguousarray(W.T)
    say("gemv_tree decode 16x4096x4096: oracle")
    ref = f32_bits(oracle.gemv_tree(x, WT, threads=16))
    return x, WT, ref, dev_bf16(x), dev_bf16(WT)


def test_decode_full_size_every_M(g, decode):
    x, WT, ref, dx, dWT = decode
    for M in range(1, 17):
        say(f"gemv_tree decode M={M}")
        got = host_bits(g.gemv_tree(dx[:M], dWT))
        assert np.array_equal(got, ref[:M]), f"M={M}: {np.count_nonzero(got != ref[:M])} outputs differ"


def test_row_content_at_any_position(g, decode):
    x, WT, ref, dx, dWT = decode
    for M, pos in ((4, 0), (8, 5), (16, 15), (3, 2)):
        B = x[:M].copy()
        B[pos] = x[9]
        got = host_bits(g.gemv_tree(dev_bf16(B), dWT))
        assert np.array_equal(got[pos], ref[9]), (M, pos)


@pytest.mark.parametrize("N,K", [(11008, 4096), (4096, 11008)])
def test_7b_decode_shapes(g, N, K):
    """The up- and down-projection decode shapes of a 7B layer (the persistent form at K = 4096, the
    one-group form at K = 11008), every row of M = 1 and M = 8 against the oracle."""
    x = synth.normal_bf16(7, f"tree7b.x{K}", (8, K))
    WT = synth.normal_bf16(7, f"tree7b.WT{N}x{K}", (N, K), 0.02)
    say(f"gemv_tree 7B shape N={N} K={K}: oracle")
    ref = f32_bits(oracle.gemv_tree(x, WT, threads=16))
    dx, dWT = dev_bf16(x), dev_bf16(WT)
    for M in (1, 8):
        got = host_bits(g.gemv_tree(dx[:M], dWT))
        assert np.array_equal(got, ref[:M]), (N, K, M, int(np.count_nonzero(got != ref[:M])))


@pytest.mark.parametrize("M,N,K", [
    (1, 1, 1), (1, 7, 8), (2, 9, 2047), (3, 13, 2048), (5, 100, 2049), (8, 4095, 4096), (16, 33, 4100),
    (4, 17, 6144), (9, 5, 6152), (16, 3, 777), (7, 600, 16392), (1, 1000, 3),
])
def test_ragged_shapes(g, M, N, K):
    x = synth.normal_bf16(M * 7 + N + K, "tree.x", (M, K))
    WT = synth.normal_bf16(M * 7 + N + K, "tree.WT", (N, K), 0.02)
    say(f"gemv_tree ragged M={M} N={N} K={K}")
    ref = f32_bits(oracle.gemv_tree(x, WT, threads=8))
    assert np.array_equal(host_bits(g.gemv_tree(dev_bf16(x), dev_bf16(WT))), ref)


def test_strided_and_misaligned_views(g):
    import torch
    xb = synth.normal_bf16(11, "tree.sx", (10, 1100))
    Wb = synth.normal_bf16(11, "tree.sW", (300, 1100), 0.02)
    dx, dW = dev_bf16(xb), dev_bf16(Wb)
    # misaligned bases and odd strides: the narrow loads
    xv, Wv = xb[1:9, 3:1003], Wb[5:290, 3:1003]
    ref = f32_bits(oracle.gemv_tree(np.ascontiguousarray(xv), np.ascontiguousarray(Wv)))
    assert np.array_equal(host_bits(g.gemv_tree(dx[1:9, 3:1003], dW[5:290, 3:1003])), ref)
    # aligned bases, strides multiples of 8 wider than K: the wide loads
    xa, Wa = xb[:, :1000], Wb[:, :1000]
    ref = f32_bits(oracle.gemv_tree(np.ascontiguousarray(xa), np.ascontiguousarray(Wa)))
    assert np.array_equal(host_bits(g.gemv_tree(dx[:, :1000], dW[:, :1000])), ref)
    # output with a row stride wider than N; the gap stays untouched
    ybig = torch.full((10, 320), float("nan"), device="cuda")
    g.gemv_tree(dx[:, :1000], dW[:, :1000], y=ybig[:, 7:307])
    assert np.array_equal(host_bits(ybig[:, 7:307].contiguous()), ref)
    assert torch.isnan(ybig[:, :7]).all() and torch.isnan(ybig[:, 307:]).all()


@pytest.mark.parametrize("name", sorted(PROBES))
def test_order_probes(g, name):
    placed, K, weights, want = PROBES[name]
    x, wt = probe(placed, K, weights)
    got = g.gemv_tree(dev_bf16(x), dev_bf16(wt))
    assert host_bits(got)[0, 0] == f32_bits(np.array([want]))[0], (name, float(got[0, 0]), want)


def test_positive_zero_and_empty(g):
    import torch
    x, wt = probe({k: -1.0 for k in range(40)}, 40, {k: 0.0 for k in range(40)})
    assert host_bits(g.gemv_tree(dev_bf16(x), dev_bf16(wt)))[0, 0] == 0
    y = torch.full((3, 5), float("nan"), device="cuda")
    g.gemv_tree(dev_bf16(np.zeros((3, 0), np.uint16)), dev_bf16(np.zeros((5, 0), np.uint16)), y=y)
    assert (host_bits(y) == 0).all()
    out = g.gemv_tree(dev_bf16(np.zeros((0, 8), np.uint16)), dev_bf16(np.zeros((5, 8), np.uint16)))
    assert tuple(out.shape) == (0, 5)


def test_rejects_more_than_16_rows(g):
    with pytest.raises(g.GGOError, match="exceeds"):
        g.gemv_tree(dev_bf16(np.zeros((17, 8), np.uint16)), dev_bf16(np.zeros((4, 8), np.uint16)))
