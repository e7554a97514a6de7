"""GPU parity of the fused epilogue: gemv_tree_ep and gemm_mfma_invariant_ep against the oracle's fold
followed by its epilogue, bit for bit (binary32 and bfloat16 outputs, every activation, with and
without bias and residual), plus a sweep of the activations over chosen binary32 values."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import dev_bf16, dev_f32, f32_bits, say

pytestmark = pytest.mark.gpu

ACTS = ["none", "relu", "silu", "gelu_tanh"]


@pytest.fixture(scope="module")
def g():
    import gemv_gemm_ordered_amd as g
    return g


def host(t):
    import torch
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().numpy().view(np.uint32)


def ref_bits(Y, bias, act, res, out):
    o = oracle.epilogue(Y, bias=bias, act=act, residual=res, out=out)
    return o if out == "bf16" else o.view(np.uint32)


def same(got, ref, out):
    """Bitwise, except that any two NaNs match (their payloads are not part of the contract)."""
    if out == "bf16":
        nan_g = (got & 0x7fff) > 0x7f80
        nan_r = (ref & 0x7fff) > 0x7f80
    else:
        nan_g = (got & 0x7fffffff) > 0x7f800000
        nan_r = (ref & 0x7fffffff) > 0x7f800000
    return np.array_equal(nan_g, nan_r) and np.array_equal(got[~nan_g], ref[~nan_r])


def sweep_values():
    v = np.concatenate([np.linspace(-110, 110, 40001, dtype=np.float32),
                        np.linspace(-2, 2, 20001, dtype=np.float32),
                        np.float32([0.0, -0.0, 1e-40, -1e-40, 1e-30, -1e-30, 3.4e38, -3.4e38, np.inf, -np.inf]),
                        synth.normal_f32(5, "epi.sweep", (4000,), 30.0)])
    return v.astype(np.float32)


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_activation_sweep_through_bias(g, act, out):
    # zero operands make every fold +0, so v = 0 + bias[n] = bias[n] (for bias = -0 it is +0) and the
    # epilogue is exercised on each chosen value
    vals = sweep_values()
    N = vals.size
    bias = dev_f32(vals)
    Y0 = np.zeros((2, N), np.float32)
    ref = ref_bits(Y0, vals, act, None, out)
    x = dev_bf16(np.zeros((2, 8), np.uint16))
    WT = dev_bf16(np.zeros((N, 8), np.uint16))
    got = host(g.gemv_tree_ep(x, WT, bias=bias, act=act, out=out))
    assert same(got, ref, out), f"gemv_tree_ep {act} {out}"
    W = dev_bf16(np.zeros((8, N), np.uint16))
    got = host(g.gemm_mfma_invariant_ep(x, W, bias=bias, act=act, out=out))
    assert same(got, ref, out), f"gemm_mfma_invariant_ep {act} {out}"


@pytest.fixture(scope="module")
def decode():
    x, W, _ = synth.decode_gemv(2, m_max=8)
    WT = np.ascontiguousarray(W.T)
    say("epilogue decode: oracle fold")
    Y = oracle.gemv_tree(x, WT, threads=16)
    bias = synth.normal_f32(2, "epi.bias", (4096,), 1.0)
    res = synth.normal_f32(2, "epi.res", (8, 4096), 1.0)
    return x, WT, Y, bias, res, dev_bf16(x), dev_bf16(WT), dev_f32(bias), dev_f32(res)


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("with_bias,with_res", [(True, True), (False, False), (True, False), (False, True)])
def test_gemv_tree_ep_decode(g, decode, act, out, with_bias, with_res):
    x, WT, Y, bias, res, dx, dWT, dbias, dres = decode
    ref = ref_bits(Y, bias if with_bias else None, act, res if with_res else None, out)
    got = host(g.gemv_tree_ep(dx, dWT, bias=dbias if with_bias else None, act=act,
                              residual=dres if with_res else None, out=out))
    assert same(got, ref, out)
    # a row's bits do not move with M
    for M in (1, 3):
        gm = host(g.gemv_tree_ep(dx[:M], dWT, bias=dbias if with_bias else None, act=act,
                                 residual=dres[:M] if with_res else None, out=out))
        assert np.array_equal(gm, got[:M]), M


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape,view", [((128, 768, 768), False), ((37, 333, 129), False), ((64, 500, 600), True)])
def test_gemm_mfma_ep_bits(g, act, out, shape, view):
    M, N, K = shape
    A = synth.normal_bf16(M + N + K, "epi.A", (M, K + 3))
    W = synth.normal_bf16(M + N + K, "epi.W", (K, N + 5), 0.02)
    bias = synth.normal_f32(M + N, "epi.mb", (N,), 0.5)
    res = synth.normal_f32(M + N, "epi.mr", (M, N), 0.5)
    if view:   # misaligned strided operands: the 128x128 instance
        Ah, Wh = A[:, 3:3 + K], W[:, 5:5 + N]
        dA, dW = dev_bf16(A)[:, 3:3 + K], dev_bf16(W)[:, 5:5 + N]
    else:
        Ah, Wh = np.ascontiguousarray(A[:, :K]), np.ascontiguousarray(W[:, :N])
        dA, dW = dev_bf16(Ah), dev_bf16(Wh)
    Y = oracle.gemm_mfma(np.ascontiguousarray(Ah), np.ascontiguousarray(Wh), threads=16)
    ref = ref_bits(Y, bias, act, res, out)
    got = host(g.gemm_mfma_invariant_ep(dA, dW, bias=dev_f32(bias), act=act, residual=dev_f32(res), out=out))
    assert same(got, ref, out)


def test_empty_k_goes_through_the_epilogue(g):
    bias = synth.normal_f32(7, "epi.k0", (40,), 3.0)
    ref = ref_bits(np.zeros((3, 40), np.float32), bias, "silu", None, "bf16")
    got = host(g.gemv_tree_ep(dev_bf16(np.zeros((3, 0), np.uint16)), dev_bf16(np.zeros((40, 0), np.uint16)),
                              bias=dev_f32(bias), act="silu", out="bf16"))
    assert np.array_equal(got, ref)
    got = host(g.gemm_mfma_invariant_ep(dev_bf16(np.zeros((3, 0), np.uint16)), dev_bf16(np.zeros((0, 40), np.uint16)),
                                        bias=dev_f32(bias), act="silu", out="bf16"))
    assert np.array_equal(got, ref)


def test_bad_epilogue_rejected(g):
    import ctypes as ct
    e = g.Epilogue(None, None, 0, 9, g.GGO_F32)
    assert g.lib.gemv_tree_ep(1, 8, 1, 8, ct.byref(e), 1, 8, 1, 8, 8, None) == -1
    e = g.Epilogue(None, None, 0, 1, 7)
    assert g.lib.gemm_mfma_invariant_ep(1, 8, 1, 8, ct.byref(e), 1, 8, 1, 8, 8, None) == -1
    e = g.Epilogue(None, 1, 4, 0, g.GGO_F32)     # residual row stride below N
    assert g.lib.gemv_tree_ep(1, 8, 1, 8, ct.byref(e), 1, 8, 1, 8, 8, None) == -1


_FOLDS = {}


@pytest.mark.parametrize("act", ["silu", "gelu_tanh"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape,tile", [((96, 2048, 1024), "128x128"), ((200, 1032, 2048), "256x128"),
                                        ((70, 4096, 4096), "256x256")])
def test_gemm_mfma_ep_on_the_wide_tiles(g, act, out, shape, tile):
    """The fused epilogue of each direct-to-LDS tile the weight rule picks (ragged M, and a ragged N for
    256x128): its passes stage a wave's rows through LDS, one to four per tile height."""
    M, N, K = shape
    if shape not in _FOLDS:
        A = synth.normal_bf16(M + K, "epiw.A", (M, K))
        W = synth.normal_bf16(N + K, "epiw.W", (K, N), 0.02)
        say(f"epilogue {tile}: oracle fold {M}x{N}x{K}")
        _FOLDS[shape] = (A, W, oracle.gemm_mfma(A, W, threads=16), synth.normal_f32(M + N, "epiw.b", (N,), 0.5),
                         synth.normal_f32(M + N, "epiw.r", (M, N), 0.5))
    A, W, Y, bias, res = _FOLDS[shape]
    ref = ref_bits(Y, bias, act, res, out)
    dA, dW = dev_bf16(A), dev_bf16(W)
    got = host(g.gemm_mfma_invariant_ep(dA, dW, bias=dev_f32(bias), act=act, residual=dev_f32(res), out=out))
    assert same(got, ref, out), (tile, act, out)
    # and the tile's plain fold (no epilogue), forced through the hook, is the oracle's fold
    assert np.array_equal(host(g.test_gemm_mfma_tile(tile if tile != "128x128" else "128x128_lds", dA, dW)),
                          f32_bits(Y)), tile
