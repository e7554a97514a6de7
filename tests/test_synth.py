"""The seeded generator: determinism, prefix property, distributions, rounding."""
import json
import os

import numpy as np

import synth
from tests.golden.make_synth_digests import digests


def test_golden_digests():
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "synth_sha256.json")))
    assert digests() == gold


def test_row_prefix_property():
    big = synth.normal_bf16(3, "x", (64, 100))
    assert np.array_equal(synth.normal_bf16(3, "x", (5, 100)), big[:5])
    assert np.array_equal(synth.normal_bf16(3, "x", (64, 100), chunk=777), big)


def test_distribution_and_rounding():
    v = synth.bf16_bits_to_f32(synth.normal_bf16(0, "d", (1 << 18,), 0.02)).astype(np.float64)
    assert abs(v.mean()) < 2e-4 and abs(v.std() - 0.02) < 2e-4
    f = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8 + 2 ** -20)], dtype=np.float32)
    assert list(synth.f32_to_bf16_bits(f)) == [0x3F80, 0x3F80, 0x3F82, 0xBF81]
    r = synth.rademacher(0, "r", 10000)
    assert set(np.unique(r)) == {-1, 1} and abs(r.mean()) < 0.05


def test_softmax_rows():
    P = synth.softmax_rows_f32(0, "p", 7, 300)
    assert P.dtype == np.float32 and (P > 0).all()
    assert np.allclose(P.astype(np.float64).sum(1), 1.0, atol=1e-6)
    assert np.array_equal(synth.softmax_rows_f32(0, "p", 3, 300, row_start=4), P[4:7])
