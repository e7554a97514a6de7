"""Pins of the oracle's Freivalds certificate ("Same Bits on the CPU and the GPU",
section "The CPU as a checker: a float Freivalds certificate").

* s = W r is exact in binary64 for these data (checked against math.fsum, which
  returns the correctly rounded exact sum);
* honest outputs of the ordered fold pass with the frozen constant 0.125, which
  must be at least twice the largest honest ratio on a calibration seed and
  hold on a second seed;
* a single planted fault of +0.005 or +0.05 is caught, and moves the residual
  by exactly the planted amount (|r_j| = 1);
* a pair of equal planted faults escapes exactly when r_j1 = -r_j2, which has
  probability 1/2 over r.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from tests.emulate import widen

C_F = 0.125


@pytest.fixture(scope="module")
def gemv_case():
    rows = 32
    x = synth.normal_bf16(0, "gemv.x", (rows, 4096), 1.0)
    _, W, r = synth.decode_gemv(0, 1)
    y = oracle.gemm_ordered(x, W, threads=8)
    return x, W, r, y, oracle.freivalds_prepare(W, r)


def test_s_is_exact(gemv_case):
    x, W, r, y, (s, q, a) = gemv_case
    wf = widen(W).astype(np.float64)
    for k in range(0, 4096, 37):
        assert s[k] == math.fsum(wf[k] * r)
        assert a[k] == pytest.approx(math.fsum(np.abs(wf[k])), rel=1e-15)
        assert q[k] == pytest.approx(math.sqrt(math.fsum(wf[k] ** 2)), rel=1e-15)


def test_honest_rows_pass_and_calibration(gemv_case):
    x, W, r, y, prep = gemv_case
    ratios = []
    for m in range(x.shape[0]):
        ok, rho, sigma, tau, bound = oracle.freivalds_check(prep, r, x[m], y[m], C_F)
        assert ok
        assert rho <= bound           # the rigorous bound is never violated by an honest row
        ratios.append(rho / sigma)
    assert C_F >= 2 * max(ratios), max(ratios)
    # validation seed
    x1, W1, r1 = synth.decode_gemv(1, 16)
    y1 = oracle.gemm_ordered(x1, W1, threads=8)
    p1 = oracle.freivalds_prepare(W1, r1)
    assert all(oracle.freivalds_check(p1, r1, x1[m], y1[m], C_F)[0] for m in range(16))


@pytest.mark.parametrize("delta", [0.005, 0.05, -0.005])
def test_single_planted_fault_is_caught(gemv_case, delta):
    x, W, r, y, prep = gemv_case
    j = int(synth.bits64(synth.stream_key(0, "fault.j"), 0, 1)[0] % 4096)
    for m in range(4):
        yb = y[m].copy()
        yb[j] = np.float32(float(yb[j]) + delta)
        ok0, rho0, *_ = oracle.freivalds_check(prep, r, x[m], y[m], C_F)
        ok, rho, sigma, tau, _ = oracle.freivalds_check(prep, r, x[m], yb, C_F)
        assert ok0 and not ok
        planted = float(yb[j]) - float(y[m][j])     # the fault as stored in binary32
        assert abs(rho - abs(planted)) <= rho0 + 1e-12   # rho = |e + r_j * delta| with |e| = rho0


def test_cancelling_pair_escape_rate_is_half():
    K = N = 128
    W = synth.normal_bf16(7, "small.W", (K, N), 0.02)
    x = synth.normal_bf16(7, "small.x", (1, K), 1.0)
    y = oracle.gemm_ordered(x, W)[0]
    trials, escaped = 1000, 0
    for t in range(trials):
        r = synth.rademacher(t, "escape.r", N)
        prep = oracle.freivalds_prepare(W, r)
        yb = y.copy()
        yb[3] += np.float32(0.05)
        yb[77] += np.float32(0.05)
        escaped += oracle.freivalds_check(prep, r, x[0], yb, C_F)[0]
        # exactly the sign rule: the pair escapes iff the two signs differ
        assert oracle.freivalds_check(prep, r, x[0], yb, C_F)[0] == (r[3] != r[77])
    # binomial(1000, 1/2): 3 sigma is 0.047
    assert abs(escaped / trials - 0.5) <= 0.047
