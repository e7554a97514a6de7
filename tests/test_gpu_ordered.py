"""GPU parity of the ordered path: gemm_ordered, gemv_ordered and the grouped
value product, bit for bit against the CPU oracle on the same seeded inputs,
plus row invariance across M and the edge cases (ragged, strided, misaligned,
empty)."""
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
def gpt2():
    A, W = synth.gpt2_projection(0, 512)
    return A, W, f32_bits(oracle.gemm_ordered(A, W, threads=8)), dev_bf16(A), dev_bf16(W)


def test_gpt2_projection_every_M_1_to_512(g, gpt2):
    A, W, ref, dA, dW = gpt2
    say("gemm_ordered gpt2 M=1..512")
    for M in range(1, 513):
        C = g.gemm_ordered(dA[:M], dW)
        got = host_bits(C)
        assert np.array_equal(got, ref[:M]), f"M={M}: {np.count_nonzero(got != ref[:M])} outputs differ"


def test_row_content_at_any_position(g, gpt2):
    A, W, ref, dA, dW = gpt2
    for pos in (0, 1, 63, 64, 100):
        B = A[:128].copy()
        B[pos] = A[300]
        got = host_bits(g.gemm_ordered(dev_bf16(B), dW))
        assert np.array_equal(got[pos], ref[300])


def test_mlp_up_full(g):
    A, W = synth.mlp_up(0, 2048)
    say("gemm_ordered mlp M=2048 oracle")
    ref = f32_bits(oracle.gemm_ordered(A, W, threads=16))
    dA, dW = dev_bf16(A), dev_bf16(W)
    for M in (64, 128, 256, 512, 1024, 2048):
        got = host_bits(g.gemm_ordered(dA[:M], dW))
        assert np.array_equal(got, ref[:M]), M


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (37, 333, 129), (65, 65, 65), (130, 70, 33), (3, 200, 1000), (64, 64, 32)])
@pytest.mark.parametrize("a_dtype", ["bf16", "f32"])
def test_ragged_shapes(g, M, N, K, a_dtype):
    Af = synth.normal_f32(M + N + K, "rag.A", (M, K))
    A = synth.f32_to_bf16_bits(Af) if a_dtype == "bf16" else Af
    W = synth.normal_bf16(M + N + K, "rag.W", (K, N), 0.02)
    ref = f32_bits(oracle.gemm_ordered(A, W))
    dA = dev_bf16(A) if a_dtype == "bf16" else dev_f32(A)
    assert np.array_equal(host_bits(g.gemm_ordered(dA, dev_bf16(W))), ref)


@pytest.mark.parametrize("M,N,K", [(37, 1100, 1001), (70, 2048, 1000), (5, 1056, 1992), (130, 1040, 1016),
                                   (37, 2100, 2001), (70, 4096, 1032), (3, 2056, 2048), (129, 2053, 2047)])
def test_ragged_shapes_on_the_64x32_and_64x64_tiles(g, M, N, K):
    """Weights of 2^20 < N K <= 2^22 elements take the 64 x 32 tile, larger ones the 64 x 64 tile: their
    element loads (odd K or N) and, with K and N multiples of 8, their wide loads with a partial last
    k-step (K not a multiple of 32)."""
    A = synth.normal_bf16(M + N + K, "rag64.A", (M, K))
    W = synth.normal_bf16(M + N + K, "rag64.W", (K, N), 0.02)
    assert N * K > 1 << 20
    say(f"gemm_ordered {'64x32' if N * K <= 1 << 22 else '64x64'} tile ragged M={M} N={N} K={K}")
    ref = f32_bits(oracle.gemm_ordered(A, W, threads=8))
    assert np.array_equal(host_bits(g.gemm_ordered(dev_bf16(A), dev_bf16(W))), ref)


TILES = ("64x64", "64x32", "16x16")


def test_every_tile_gives_the_same_bits(g, gpt2):
    """The tile is a speed knob ("Taming Bitwise Behavior in GPU Kernels with Tensor Core", section 3.2.2):
    each of the three tiles, forced on the same rows at the same M, gives the oracle's bits."""
    A, W, ref, dA, dW = gpt2
    for M in (1, 7, 64, 130, 512):
        for tile in TILES:
            say(f"gemm_ordered tile {tile} gpt2 M={M}")
            assert np.array_equal(host_bits(g.test_gemm_ordered_tile(tile, dA[:M], dW)), ref[:M]), (tile, M)
    Am, Wm = synth.mlp_up(5, 256)
    refm = f32_bits(oracle.gemm_ordered(Am, Wm, threads=16))
    dAm, dWm = dev_bf16(Am), dev_bf16(Wm)
    for tile in TILES:
        say(f"gemm_ordered tile {tile} mlp M=256")
        assert np.array_equal(host_bits(g.test_gemm_ordered_tile(tile, dAm, dWm)), refm), tile


@pytest.mark.parametrize("M,N,K", [(37, 333, 129), (5, 70, 1000), (66, 130, 64)])
@pytest.mark.parametrize("a_dtype", ["bf16", "f32"])
def test_every_tile_on_ragged_shapes(g, M, N, K, a_dtype):
    Af = synth.normal_f32(M + N + K, "ragt.A", (M, K))
    A = synth.f32_to_bf16_bits(Af) if a_dtype == "bf16" else Af
    W = synth.normal_bf16(M + N + K, "ragt.W", (K, N), 0.02)
    ref = f32_bits(oracle.gemm_ordered(A, W))
    dA = dev_bf16(A) if a_dtype == "bf16" else dev_f32(A)
    dW = dev_bf16(W)
    for tile in TILES:
        assert np.array_equal(host_bits(g.test_gemm_ordered_tile(tile, dA, dW)), ref), tile
    # misaligned views take the element loads of every tile
    dAb = dev_bf16(np.pad(A, ((0, 0), (1, 0)))) if a_dtype == "bf16" else dev_f32(np.pad(A, ((0, 0), (1, 0))))
    for tile in TILES:
        assert np.array_equal(host_bits(g.test_gemm_ordered_tile(tile, dAb[:, 1:], dW)), ref), tile


def test_strided_and_misaligned_views(g):
    A, W = synth.mlp_up(4, 96)
    # row strides not multiples of 8, base pointers off 16-byte alignment
    Av, Wv = A[1:90, 3:1003], np.ascontiguousarray(W[3:1003, :])[:, 5:400]
    ref = f32_bits(oracle.gemm_ordered(np.ascontiguousarray(Av), np.ascontiguousarray(Wv)))
    dA, dW = dev_bf16(A), dev_bf16(np.ascontiguousarray(W[3:1003, :]))
    got = g.gemm_ordered(dA[1:90, 3:1003], dW[:, 5:400])
    assert np.array_equal(host_bits(got), ref)
    # output with a row stride wider than N
    import torch
    Cbig = torch.full((89, 512), float("nan"), device="cuda")
    g.gemm_ordered(dA[1:90, 3:1003], dW[:, 5:400], C=None)
    out = Cbig[:, 7:402]
    g.gemm_ordered(dA[1:90, 3:1003], dW[:, 5:400], C=out)
    assert np.array_equal(host_bits(out.contiguous()), ref)
    assert torch.isnan(Cbig[:, :7]).all() and torch.isnan(Cbig[:, 402:]).all()


def test_empty_and_zero_K(g):
    import torch
    A = torch.zeros((5, 0), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((0, 7), dtype=torch.bfloat16, device="cuda")
    C = torch.full((5, 7), 3.0, device="cuda")
    g.gemm_ordered(A, W, C=C)
    assert (host_bits(C) == 0).all()
    C2 = torch.full((5, 7), 3.0, device="cuda")
    g.gemv_ordered(A, W, y=C2)
    assert (host_bits(C2) == 0).all()
    g.gemm_ordered(torch.zeros((0, 4), dtype=torch.bfloat16, device="cuda"),
                   torch.zeros((4, 7), dtype=torch.bfloat16, device="cuda"))


def test_worked_examples_on_gpu(g):
    from tests.test_oracle_pins import GOLD, bf16_of, hexf
    w1 = GOLD["W1_order"]
    a = bf16_of([hexf(v) for v in w1["a"]])[None, :]
    w = bf16_of([hexf(v) for v in w1["w"]])[:, None]
    assert hex(host_bits(g.gemm_ordered(dev_bf16(a), dev_bf16(w)))[0, 0]) == w1["expected_bits"]
    assert hex(host_bits(g.gemv_ordered(dev_bf16(a), dev_bf16(w)))[0, 0]) == w1["expected_bits"]
    w2 = GOLD["W2_fma"]
    a = np.array([[hexf(v) for v in w2["a"]]], dtype=np.float32)
    w = bf16_of([hexf(v) for v in w2["w"]])[:, None]
    assert "0x%08x" % host_bits(g.gemm_ordered(dev_f32(a), dev_bf16(w)))[0, 0] == w2["expected_bits"]


def test_subnormals_kept_and_no_negative_zero(g):
    from tests.test_oracle_pins import bf16_of
    a = np.array([[1.0, -1.0, 2.0 ** -100, 2.0 ** -30], [2.0 ** -100, 0, 0, 0]], dtype=np.float32)
    w = bf16_of([2.0 ** -40, 2.0 ** -40, 2.0 ** -40, -2.0 ** -110])[:, None]
    ref = f32_bits(oracle.gemm_ordered(a, w))
    assert np.array_equal(host_bits(g.gemm_ordered(dev_f32(a), dev_bf16(w))), ref)
    assert ref[1, 0] != 0     # a subnormal result, kept


def test_gemv_decode_matches_oracle_and_gemm(g):
    """Every M from 1 to 16 at the decode size (M <= 4 and M > 4 take differently staged kernels)."""
    say("gemv decode x[16,4096] W[4096,4096]")
    x, W, _ = synth.decode_gemv(0, 16)
    ref = f32_bits(oracle.gemm_ordered(x, W, threads=16))
    dx, dW = dev_bf16(x), dev_bf16(W)
    for M in range(1, 17):
        y = host_bits(g.gemv_ordered(dx[:M], dW))
        assert np.array_equal(y, ref[:M]), M
    for M in (1, 4, 8):
        assert np.array_equal(host_bits(g.gemm_ordered(dx[:M], dW)), ref[:M])


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 13, 16])
@pytest.mark.parametrize("K,N", [(777, 1000), (772, 1000), (64, 16), (4, 2), (1, 1), (1092, 30), (2048, 4097),
                                 (128, 34), (256, 18), (132, 48), (384, 30)])
def test_gemv_ragged(g, M, K, N):
    # K % 4 == 0 and even N take the wide loads (edges masked), the rest element loads
    say(f"gemv ragged M={M} K={K} N={N}")
    x = synth.normal_bf16(M * 7 + K, "gv.x", (M, K))
    W = synth.normal_bf16(N + K, "gv.W", (K, N), 0.02)
    ref = f32_bits(oracle.gemm_ordered(x, W))
    assert np.array_equal(host_bits(g.gemv_ordered(dev_bf16(x), dev_bf16(W))), ref)
    # strided and misaligned
    dxb = dev_bf16(np.pad(x, ((0, 0), (1, 2))))
    dWb = dev_bf16(np.pad(W, ((0, 0), (3, 0))))
    assert np.array_equal(host_bits(g.gemv_ordered(dxb[:, 1:K + 1], dWb[:, 3:])), ref)
    # strided but aligned (row strides a multiple of 8 elements)
    dxa = dev_bf16(np.pad(x, ((0, 0), (0, 8 - K % 8 if K % 8 else 8))))
    dWa = dev_bf16(np.pad(W, ((0, 0), (0, 8 - N % 8 if N % 8 else 8))))
    assert np.array_equal(host_bits(g.gemv_ordered(dxa[:, :K], dWa[:, :N])), ref)


def test_gemv_wt_decode_every_M(g):
    """The W^T form at the decode size: every M from 1 to 16 against the oracle, and equal to gemv_ordered
    on W [K, N]."""
    say("gemv_ordered_wt decode x[16,4096] W^T[4096,4096]")
    x, W, _ = synth.decode_gemv(0, 16)
    ref = f32_bits(oracle.gemm_ordered(x, W, threads=16))
    dx, dW, dWT = dev_bf16(x), dev_bf16(W), dev_bf16(np.ascontiguousarray(W.T))
    for M in range(1, 17):
        y = host_bits(g.gemv_ordered_wt(dx[:M], dWT))
        assert np.array_equal(y, ref[:M]), M
    assert np.array_equal(host_bits(g.gemv_ordered(dx[:8], dW)), ref[:8])


@pytest.mark.parametrize("M,K,N", [(1, 4, 1), (3, 100, 17), (5, 1028, 33), (16, 4096, 4095), (2, 16392, 600),
                                   (9, 4100, 13), (8, 64, 16), (7, 772, 1000), (1, 11008, 40),
                                   (6, 128, 18), (12, 256, 31), (16, 132, 48)])
def test_gemv_wt_ragged_and_strided(g, M, K, N):
    import torch
    say(f"gemv_ordered_wt ragged M={M} K={K} N={N}")
    x = synth.normal_bf16(M * 7 + K, "gvt.x", (M, K))
    W = synth.normal_bf16(N + K, "gvt.W", (K, N), 0.02)
    ref = f32_bits(oracle.gemm_ordered(x, W))
    WT = np.ascontiguousarray(W.T)
    assert np.array_equal(host_bits(g.gemv_ordered_wt(dev_bf16(x), dev_bf16(WT))), ref)
    # row strides past K (multiples of 4), padding filled with NaN: it must never be read
    nan = np.uint16(0x7fc1)
    xp = np.full((M, K + 12), nan, dtype=np.uint16)
    xp[:, :K] = x
    wp = np.full((N, K + 4), nan, dtype=np.uint16)
    wp[:, :K] = WT
    yb = torch.full((M, N + 5), -3.0, device="cuda")
    g.gemv_ordered_wt(dev_bf16(xp)[:, :K], dev_bf16(wp)[:, :K], y=yb[:, :N])
    got = host_bits(yb)
    assert np.array_equal(got[:, :N], ref)
    assert (got[:, N:] == np.float32(-3.0).view(np.uint32)).all()


def test_gemv_wt_rejects_what_it_cannot_take(g):
    import torch
    x = torch.zeros((2, 72), dtype=torch.bfloat16, device="cuda")
    WT = torch.zeros((16, 72), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(g.GGOError):
        g.gemv_ordered_wt(x[:, :70], WT[:, :70])          # K % 4 != 0
    with pytest.raises(g.GGOError):
        g.gemv_ordered_wt(x[:, 2:66], WT[:, :64])         # x not 8-byte aligned
    with pytest.raises(g.GGOError):
        g.gemv_ordered_wt(torch.zeros((17, 64), dtype=torch.bfloat16, device="cuda"), WT[:, :64])   # M > 16


def _pv_problem(seq, L, heads=4):
    P, V = synth.pv_sequence(0, seq, L, heads=heads)
    return P, V


@pytest.mark.parametrize("L", [1, 15, 16, 64, 256])
def test_pv_solo(g, L):
    import torch
    P, V = _pv_problem(0, L)
    ref = np.stack([f32_bits(oracle.gemm_ordered(P[h], V[h])) for h in range(P.shape[0])])
    dP, dV = dev_f32(P), dev_bf16(V)
    O = torch.empty((P.shape[0], L, 128), dtype=torch.float32, device="cuda")
    g.gemm_ordered_grouped([(dP, dV, O)])
    assert np.array_equal(host_bits(O), ref)


def test_pv_mixed_batches_every_order(g):
    import torch
    lens = [15, 16, 1, 64, 256, 15, 3, 100]
    probs = [_pv_problem(i, L) for i, L in enumerate(lens)]
    refs = [np.stack([f32_bits(oracle.gemm_ordered(P[h], V[h])) for h in range(P.shape[0])]) for P, V in probs]
    dev = [(dev_f32(P), dev_bf16(V)) for P, V in probs]
    rng = np.random.default_rng(0)
    for trial in range(4):
        order = rng.permutation(len(lens)) if trial else np.arange(len(lens))
        outs = {i: torch.full((4, lens[i], 128), float("nan"), device="cuda") for i in order}
        g.gemm_ordered_grouped([(dev[i][0], dev[i][1], outs[i]) for i in order])
        for i in order:
            assert np.array_equal(host_bits(outs[i]), refs[i]), (trial, i)


def test_pv_long_sequences_sampled_rows(g):
    import torch
    for L in (1024, 5000):
        say(f"pv L={L}")
        heads = 2
        P, V = _pv_problem(1, L, heads=heads)
        dP, dV = dev_f32(P), dev_bf16(V)
        O = torch.empty((heads, L, 128), dtype=torch.float32, device="cuda")
        g.gemm_ordered_grouped([(dP, dV, O)])
        got = host_bits(O)
        rows = [0, 1, L // 2, L - 1]
        for h in range(heads):
            ref = f32_bits(oracle.gemm_ordered(np.ascontiguousarray(P[h][rows]), V[h]))
            assert np.array_equal(got[h][rows], ref), (L, h)


def _device_pv(L, heads, seed):
    """P = softmax of N(0, 1) logits (binary32, on the device) and V ~ N(0, 1) bf16 for one sequence of the
    value product at its full size; drawn with torch's seeded generator on the device, since a host draw of
    32 x 5000 x 5000 values would take minutes. Both sides read the same bytes."""
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    P = torch.softmax(torch.randn((heads, L, L), device="cuda", generator=gen), dim=-1)
    V = torch.randn((heads, L, 128), device="cuda", generator=gen).to(torch.bfloat16)
    return P, V


def _pv_rows_vs_oracle(P, V, O, rows, what):
    import torch
    torch.cuda.synchronize()
    for h in range(P.shape[0]):
        Ph = P[h, rows].cpu().numpy()
        Vh = V[h].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        ref = f32_bits(oracle.gemm_ordered(np.ascontiguousarray(Ph), Vh))
        got = O[h, rows].cpu().numpy().view(np.uint32)
        assert np.array_equal(got, ref), (what, h, rows)


def test_pv_full_size_32_heads(g):
    """The value product at the configuration's full size: 32 heads at L = 5000 (P is 3.2 GB, so the later
    heads sit more than 2^31 bytes past P's start) and 32 heads at L = 1024 in one launch, then a mixed
    batch with both among short sequences in another order; sampled rows of every head, head 31
    included, against the oracle, and each output equal bit for bit across the two launches."""
    import torch
    say("pv full size: drawing P and V on the device (L=5000 and L=1024, 32 heads)")
    P5, V5 = _device_pv(5000, 32, 50)
    P1, V1 = _device_pv(1024, 32, 51)
    P15, V15 = _device_pv(15, 32, 52)
    P16, V16 = _device_pv(16, 32, 53)
    assert P5[31].data_ptr() - P5.data_ptr() > 1 << 31     # head 31 starts past 2^31 bytes
    O5 = torch.full((32, 5000, 128), float("nan"), device="cuda")
    O1 = torch.full((32, 1024, 128), float("nan"), device="cuda")
    say("pv full size: 32 x L=5000 + 32 x L=1024 in one launch")
    g.gemm_ordered_grouped([(P5, V5, O5), (P1, V1, O1)])
    _pv_rows_vs_oracle(P5, V5, O5, [0, 1, 2500, 4998, 4999], "L=5000")
    _pv_rows_vs_oracle(P1, V1, O1, [0, 511, 1023], "L=1024")
    assert not torch.isnan(O5).any() and not torch.isnan(O1).any()
    say("pv full size: mixed batch [15, 5000, 16, 1024] in another order")
    M5, M1 = torch.empty_like(O5), torch.empty_like(O1)
    M15 = torch.empty((32, 15, 128), device="cuda")
    M16 = torch.empty((32, 16, 128), device="cuda")
    g.gemm_ordered_grouped([(P15, V15, M15), (P1, V1, M1), (P16, V16, M16), (P5, V5, M5)])
    torch.cuda.synchronize()
    assert torch.equal(M5.view(torch.int32), O5.view(torch.int32))
    assert torch.equal(M1.view(torch.int32), O1.view(torch.int32))
    _pv_rows_vs_oracle(P15, V15, M15, list(range(15)), "L=15")
    _pv_rows_vs_oracle(P16, V16, M16, list(range(16)), "L=16")
