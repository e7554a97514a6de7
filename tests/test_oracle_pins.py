"""Pins of the CPU oracle against facts that do not come from the oracle itself.

* the binary64 emulation of the binary32 fold (tests/emulate.py), bit for bit;
* exact rational dot products on tiny shapes, within the classical bound;
* hand-derived worked examples (tests/golden/worked_examples.json);
* integer data, where every summation order is exact;
* the invariants the method promises: row bits independent of M and of row position.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from tests.emulate import as_f64, bits, exact_dot, fold_f64_emulated, widen

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def hexf(s):
    return float.fromhex(s)


def bf16_of(vals):
    out = synth.f32_to_bf16_bits(np.array(vals, dtype=np.float32))
    assert (widen(out) == np.array(vals, dtype=np.float32)).all(), "value not exact in bf16"
    return out


def test_w1_ascending_order():
    g = GOLD["W1_order"]
    A = bf16_of([hexf(v) for v in g["a"]])[None, :]
    W = bf16_of([hexf(v) for v in g["w"]])[:, None]
    C = oracle.gemm_ordered(A, W)
    assert hex(bits(C)[0, 0]) == g["expected_bits"]
    # the emulator agrees, and the reversed fold is the documented other value
    assert hex(bits(fold_f64_emulated(A, W))[0, 0]) == g["expected_bits"]
    assert hex(bits(fold_f64_emulated(A, W, reverse=True))[0, 0]) == g["k_reversed_bits"]


def test_w2_separate_multiply_and_add():
    g = GOLD["W2_fma"]
    A = np.array([[hexf(v) for v in g["a"]]], dtype=np.float32)
    W = bf16_of([hexf(v) for v in g["w"]])[:, None]
    C = oracle.gemm_ordered(A, W)
    assert "0x%08x" % bits(C)[0, 0] == g["expected_bits"]
    # the contracted value, computed exactly with fractions
    from fractions import Fraction
    exact = Fraction(float(A[0, 0])) * Fraction(float(widen(W)[0, 0])) + Fraction(float(A[0, 1])) * Fraction(float(widen(W)[1, 0]))
    assert "0x%08x" % np.float32(float(exact)).view(np.uint32) == g["contracted_bits"]


@pytest.mark.parametrize("K", [8, 64, 577])
def test_w3_order_probe_pure_chain(K):
    L, r = 1024.0, 2.0 ** -15
    rows = []
    for m in range(1, K - 1):
        a = np.zeros(K, dtype=np.float32)
        a[0], a[m], a[m + 1] = r, L, -L
        rows.append(a)
    A = synth.f32_to_bf16_bits(np.array(rows))
    W = bf16_of([1.0] * K)[:, None]
    C = oracle.gemm_ordered(A, W)
    assert (bits(C) == 0).all()      # +0.0 everywhere: r absorbed by +L, then exact cancellation
    # control: with the pair cancelled before r arrives, r survives (the probe can fail)
    a = np.zeros(K, dtype=np.float32); a[0], a[1], a[K - 1] = L, -L, r
    C2 = oracle.gemm_ordered(synth.f32_to_bf16_bits(a[None]), W)
    assert C2[0, 0] == np.float32(r)


def _cases():
    A1, W1 = synth.gpt2_projection(0, 64)
    yield "gpt2_m64", A1, W1
    x, W2, _ = synth.decode_gemv(1, 8)
    yield "gemv_m8_rows", x[:2], W2[:, :512]
    A3, W3 = synth.mlp_up(2, 64)
    yield "mlp_m64", A3[:16], W3[:, :1024]
    P, V = synth.pv_sequence(0, 0, 64, heads=2)
    yield "pv_L64_f32A", P[1], V[1]


@pytest.mark.parametrize("name,A,W", list(_cases()), ids=lambda v: v if isinstance(v, str) else "")
def test_oracle_equals_f64_emulation(name, A, W):
    C = oracle.gemm_ordered(A, W)
    E = fold_f64_emulated(A, W)
    assert np.array_equal(bits(C), bits(E)), name


def test_oracle_ragged_strided_views():
    A, W = synth.mlp_up(3, 40)
    Asub = A[3:40, 5:1000]            # row stride 1024, not a multiple of the width
    Wsub = np.ascontiguousarray(W[5:1000, 7:340])
    C = oracle.gemm_ordered(Asub, Wsub)
    E = fold_f64_emulated(np.ascontiguousarray(Asub), Wsub)
    assert np.array_equal(bits(C), bits(E))


@pytest.mark.parametrize("seed", [0, 1])
def test_oracle_within_exact_bound_tiny(seed):
    rng = np.random.default_rng(seed)
    for K in (1, 2, 3, 17, 64):
        for a_dtype in ("bf16", "f32"):
            M, N = 4, 5
            Af = rng.standard_normal((M, K)).astype(np.float32)
            A = synth.f32_to_bf16_bits(Af) if a_dtype == "bf16" else Af
            W = synth.f32_to_bf16_bits(rng.standard_normal((K, N)).astype(np.float32) * 0.02)
            C = oracle.gemm_ordered(A, W)
            a, w = as_f64(A), widen(W).astype(np.float64)
            u = 2.0 ** -24
            gamma = K * u / (1 - K * u)
            for m in range(M):
                for n in range(N):
                    ex = exact_dot(a[m], w[:, n])
                    scale = float(sum(abs(a[m, k] * w[k, n]) for k in range(K)))
                    assert abs(float(ex) - float(C[m, n])) <= gamma * scale + 1e-300


def test_integer_data_every_order_exact():
    A = synth.integer_bf16(0, "int.A", (33, 300))
    W = synth.integer_bf16(0, "int.W", (300, 70))
    C = oracle.gemm_ordered(A, W)
    exact = widen(A).astype(np.int64) @ widen(W).astype(np.int64)
    assert np.array_equal(C.astype(np.int64), exact)
    assert np.array_equal(oracle.gemm_f64(A, W).astype(np.int64), exact)


def test_f64_reference_is_the_exact_sum_on_tiny_shapes():
    A, W = synth.gpt2_projection(5, 3)
    A, W = A[:, :40], np.ascontiguousarray(W[:40, :6])
    D = oracle.gemm_f64(A, W)
    S = oracle.gemm_absdot_f64(A, W)
    a, w = as_f64(A), widen(W).astype(np.float64)
    for m in range(3):
        for n in range(6):
            ex = exact_dot(a[m], w[:, n])
            assert abs(float(ex) - D[m, n]) <= 40 * 2.0 ** -53 * S[m, n]
            assert S[m, n] == pytest.approx(float(sum(abs(a[m, k] * w[k, n]) for k in range(40))), rel=1e-14)


def test_oracle_rows_independent_of_M_and_position():
    A, W = synth.gpt2_projection(0, 512)
    full = bits(oracle.gemm_ordered(A, W, threads=8))
    for M in (1, 2, 3, 7, 31, 64, 100, 257, 511):
        assert np.array_equal(bits(oracle.gemm_ordered(A[:M], W)), full[:M]), M
    # one row's content at several row positions of a batch
    row = A[17]
    for pos in (0, 5, 63):
        B = A[:64].copy()
        B[pos] = row
        assert np.array_equal(bits(oracle.gemm_ordered(B, W))[pos], full[17])


def test_oracle_never_negative_zero_with_subnormals_kept():
    # cancellations give +0; tiny subnormal partial sums survive (no flush to zero)
    a = np.array([[1.0, -1.0, 2.0 ** -100, 2.0 ** -30]], dtype=np.float32)
    w = bf16_of([1.0, 1.0, 2.0 ** -40, -2.0 ** -110])[:, None]
    C = oracle.gemm_ordered(a, w)
    expected = np.float32(2.0 ** -140) + np.float32(-(2.0 ** -140))
    assert bits(C)[0, 0] == 0 and not math.copysign(1, float(C[0, 0])) < 0
    assert expected == 0
    a2 = np.array([[2.0 ** -100]], dtype=np.float32)
    w2 = bf16_of([2.0 ** -40])[:, None]
    assert oracle.gemm_ordered(a2, w2)[0, 0] == np.float32(2.0 ** -140) != 0


def test_clopper_pearson_reading_reproduces_printed_value():
    g = GOLD["W6_clopper_pearson"]
    ub = 1 - 0.05 ** (1 / g["n"])
    assert round(100 * ub, 3) == g["printed_percent"]
