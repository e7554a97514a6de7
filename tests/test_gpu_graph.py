"""Every entry point captured in a HIP graph gives the bits of its eager call on every replay.

The decode benchmark times the GEMVs as replays of one captured graph, and a serving loop may capture
these calls too. The library's calls put kernels on the caller's stream and nothing else (no memory set or
copy nodes; a problem table travels by value as a kernel argument), so a replay has to reproduce the eager
call exactly. Each case runs the call eagerly, captures the same call into a graph, and replays the graph
three times; before each replay the output is filled with NaN by eager work on the stream, and the process
synchronises before and after the replay. Every replay must equal the eager bits. For the headline tree
GEMV the eager bits are also checked against the oracle here; the other entry points' parity with the
oracle is covered by their own tests.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import dev_bf16, dev_f32, f32_bits, say

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def g():
    import gemv_gemm_ordered_amd as g
    return g


def bits(t):
    """The output's bit patterns on the host (float32 or bfloat16)."""
    import torch
    torch.cuda.synchronize()
    return t.detach().cpu().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy().copy()


def replays_match(call, out, name):
    """Eager bits of call() in out, then REPLAYS graph replays of the captured call, each after out was
    poisoned with NaN; returns the eager bits."""
    import torch
    say(f"graph: {name}")
    torch.cuda.synchronize()
    call()
    ref = bits(out)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for i in range(REPLAYS):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = bits(out)
        assert np.array_equal(got, ref), f"{name}: replay {i} differs from the eager call in {int((got != ref).sum())} words"
    return ref


@pytest.fixture(scope="module")
def decode():
    x, W, _ = synth.decode_gemv(11, m_max=8)
    WT = np.ascontiguousarray(W.T)
    return {"x": x, "W": W, "WT": WT, "dx": dev_bf16(x), "dW": dev_bf16(W), "dWT": dev_bf16(WT),
            "tree": f32_bits(oracle.gemv_tree(x, WT, threads=16))}


@pytest.mark.parametrize("M", [1, 4, 8])
def test_tree_gemv_decode(g, decode, M):
    import torch
    y = torch.empty((M, 4096), dtype=torch.float32, device="cuda")
    ref = replays_match(lambda: g.gemv_tree(decode["dx"][:M], decode["dWT"], y=y), y, f"gemv_tree M={M} 4096x4096")
    assert np.array_equal(ref.view(np.uint32), decode["tree"][:M]), "eager tree GEMV differs from the oracle"


def test_tree_gemv_one_group_form(g):
    import torch
    M, N, K = 3, 1000, 777   # K not a multiple of 8: the one-group form
    x = synth.normal_bf16(12, "graph.x", (M, K), 1.0)
    WT = synth.normal_bf16(12, "graph.WT", (N, K), 0.02)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    dx, dWT = dev_bf16(x), dev_bf16(WT)
    ref = replays_match(lambda: g.gemv_tree(dx, dWT, y=y), y, "gemv_tree 3x1000x777")
    assert np.array_equal(ref.view(np.uint32), f32_bits(oracle.gemv_tree(x, WT))), "eager tree GEMV differs from the oracle"


def test_tree_gemv_fused_epilogue(g, decode):
    import torch
    M, N = 4, 4096
    bias = dev_f32(synth.normal_f32(13, "graph.bias", (N,), 0.1))
    res = dev_f32(synth.normal_f32(13, "graph.res", (M, N), 1.0))
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    replays_match(lambda: g.gemv_tree_ep(decode["dx"][:M], decode["dWT"], bias=bias, act="silu", residual=res,
                                         out="bf16", y=y), y, "gemv_tree_ep M=4 silu, bias, residual, bf16 out")


def test_matrix_core_gemv(g, decode):
    import torch
    y = torch.empty((8, 4096), dtype=torch.float32, device="cuda")
    replays_match(lambda: g.gemv_mfma_invariant(decode["dx"], decode["dWT"], y=y), y, "gemv_mfma_invariant M=8")


@pytest.mark.parametrize("M", [1, 8])
def test_ordered_gemv_wt(g, decode, M):
    import torch
    y = torch.empty((M, 4096), dtype=torch.float32, device="cuda")
    replays_match(lambda: g.gemv_ordered_wt(decode["dx"][:M], decode["dWT"], y=y), y, f"gemv_ordered_wt M={M}")


def test_ordered_gemv_kn(g, decode):
    import torch
    y = torch.empty((4, 4096), dtype=torch.float32, device="cuda")
    replays_match(lambda: g.gemv_ordered(decode["dx"][:4], decode["dW"], y=y), y, "gemv_ordered M=4 W [K, N]")


@pytest.mark.parametrize("which,M", [("gpt2", 8), ("mlp", 256)])
def test_ordered_gemm(g, which, M):
    import torch
    A, W = synth.gpt2_projection(14, m_max=M) if which == "gpt2" else synth.mlp_up(14, m_max=M)
    dA, dW = dev_bf16(A), dev_bf16(W)
    C = torch.empty((M, W.shape[1]), dtype=torch.float32, device="cuda")
    replays_match(lambda: g.gemm_ordered(dA, dW, C=C), C, f"gemm_ordered {which} M={M}")


def test_ordered_gemm_empty_k(g):
    import torch
    dA = torch.empty((5, 0), dtype=torch.bfloat16, device="cuda")
    dW = torch.empty((0, 7), dtype=torch.bfloat16, device="cuda")
    C = torch.empty((5, 7), dtype=torch.float32, device="cuda")
    ref = replays_match(lambda: g.gemm_ordered(dA, dW, C=C), C, "gemm_ordered K=0")
    assert np.array_equal(ref, np.zeros((5, 7), dtype=np.int32)), "K = 0 must give +0.0 everywhere"


def test_value_product_grouped(g):
    import torch
    P, V = synth.pv_sequence(15, 0, 64, heads=2)
    dP, dV = dev_f32(P), dev_bf16(V)
    O = torch.empty((2, 64, 128), dtype=torch.float32, device="cuda")
    replays_match(lambda: g.gemm_ordered_grouped([(dP, dV, O)]), O, "gemm_ordered_grouped P.V 2 heads L=64")


def test_matrix_core_gemm(g):
    import torch
    A, W = synth.mlp_up(16, m_max=256)
    dA, dW = dev_bf16(A), dev_bf16(W)
    C = torch.empty((256, 4096), dtype=torch.float32, device="cuda")
    replays_match(lambda: g.gemm_mfma_invariant(dA, dW, C=C), C, "gemm_mfma_invariant mlp M=256")
