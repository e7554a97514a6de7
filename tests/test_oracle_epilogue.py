"""Pins for the oracle's fused epilogue (``oracle_epilogue``, ``oracle_ep_exp``).

The epilogue's order (bias, activation, residual, then the output type) and its activations are this
library's definitions (the pages name none). Each function is pinned against the mathematics it
approximates, or against values that fix it exactly:
  * exp: within 2 units in the last place of the binary32 result, on a dense grid and at the ends of
    its range (a wrong coefficient, a dropped term or a wrong reduction constant breaks this);
  * relu, the order of the steps and the bf16 rounding: exact values worked out by hand;
  * silu and gelu: within a stated bound of their binary64 definitions.
The mutant gates at the end check that the pins catch a planted change of each part.
"""
import hashlib
import math
import os
import shutil

import numpy as np
import pytest

import oracle
from oracle import build as obuild


def f32(x):
    return np.float32(x)


def ulp(x):
    x = abs(float(np.float32(x)))
    if x == 0 or not math.isfinite(x):
        return 2.0 ** -149
    return max(float(np.spacing(np.float32(x))), 2.0 ** -149)


def test_exp_exact_points():
    assert oracle.ep_exp(0.0) == 1.0
    assert oracle.ep_exp(-0.0) == 1.0
    assert oracle.ep_exp(100.0) == math.inf
    assert oracle.ep_exp(-200.0) == 0.0
    assert oracle.ep_exp(-math.inf) == 0.0 and oracle.ep_exp(math.inf) == math.inf
    assert math.isnan(oracle.ep_exp(math.nan))


def test_exp_within_two_ulp():
    xs = np.concatenate([np.linspace(-87.0, 88.7, 200001, dtype=np.float32),
                         np.float32([1e-8, -1e-8, 0.3465736, -0.3465736, 88.72, -87.33])])
    worst = 0.0
    for x in xs:
        x = float(x)
        e = oracle.ep_exp(x)
        ref = math.exp(x)            # x is exactly the binary32 input
        worst = max(worst, abs(e - ref) / ulp(ref))
    assert worst <= 2.0, worst


def test_exp_subnormal_range_monotone_and_close():
    xs = np.linspace(-103.9, -87.4, 5001, dtype=np.float32)
    vals = [oracle.ep_exp(float(x)) for x in xs]
    assert all(a <= b for a, b in zip(vals, vals[1:]))
    for x, v in zip(xs, vals):
        assert abs(v - math.exp(float(x))) <= 2 * 2.0 ** -149 + 2 * ulp(math.exp(float(x)))


def ep(y, **kw):
    return oracle.epilogue(np.array([[y]], dtype=np.float32), **kw)[0, 0]


def test_relu_exact():
    for v, want in ((1.5, 1.5), (-1.5, 0.0), (0.0, 0.0), (-0.0, 0.0), (1e-40, 1e-40), (-1e-40, 0.0)):
        got = ep(v, act="relu")
        assert got == f32(want) and not math.copysign(1.0, float(got)) < 0, (v, got)


def test_order_bias_then_act_then_residual():
    # y = 1, bias = -2, residual = -1 with relu: relu(1 - 2) + (-1) = -1. Other orders give
    # relu(1 - 2 - 1) = 0, relu(1) - 2 - 1 = -2 and relu(1 - 1) - 2 = -2.
    got = oracle.epilogue(np.array([[1.0]], np.float32), bias=np.array([-2.0], np.float32), act="relu",
                          residual=np.array([[-1.0]], np.float32))[0, 0]
    assert got == -1.0


def test_bf16_rounding_exact():
    def bf(u):
        v = np.array([[u]], dtype=np.uint32).view(np.float32)
        return int(oracle.epilogue(v, out="bf16")[0, 0])
    assert bf(0x3f808000) == 0x3f80      # tie, even stays
    assert bf(0x3f818000) == 0x3f82      # tie, odd rounds up
    assert bf(0x3f80ffff) == 0x3f81
    assert bf(0x3f807fff) == 0x3f80
    assert bf(0xbf818000) == 0xbf82      # sign-magnitude
    assert bf(0x7f7fffff) == 0x7f80      # rounds up to infinity
    assert bf(0x7f800000) == 0x7f80
    assert bf(0x7fc00001) == 0x7fc0      # NaN
    assert bf(0x00008000) == 0x0000      # subnormal tie to even (zero)


@pytest.mark.parametrize("act", ["silu", "gelu_tanh"])
def test_activations_close_to_binary64(act):
    # Each of these is a short chain of binary32 steps around one exp (<= 2 ulp), so the result lies
    # within 8 ulp of the binary64 value, plus an absolute 2^-22 |v| where a difference (1 + tanh, for
    # large negative v) cancels.
    vs = np.concatenate([np.linspace(-30, 30, 60001, dtype=np.float32), np.float32([1e-30, -1e-30, 1e-3, -1e-3])])
    out = oracle.epilogue(vs[None, :], act=act)[0]
    for v, g in zip(vs.astype(np.float64), out.astype(np.float64)):
        if act == "silu":
            ref = v / (1.0 + math.exp(-v))
        else:
            u = math.sqrt(2 / math.pi) * (v + 0.044715 * v ** 3)
            ref = 0.5 * v * (1.0 + math.tanh(u))
        assert abs(g - ref) <= 8 * ulp(ref) + 2.0 ** -22 * abs(v), (act, v, g, ref)


def test_special_values():
    assert ep(0.0, act="silu") == 0.0 and ep(0.0, act="gelu_tanh") == 0.0
    assert ep(1e30, act="silu") == f32(1e30) and ep(1e30, act="gelu_tanh") == f32(1e30)
    assert ep(-1e30, act="silu") == 0.0 and ep(-1e30, act="gelu_tanh") == 0.0


# ---- mutant gates ----

MUTANTS = {
    "residual_before_act": ("            v = ep_act(v, act);\n            if (residual)\n                v = v + residual[m * ldr + n];",
                            "            if (residual)\n                v = v + residual[m * ldr + n];\n            v = ep_act(v, act);"),
    "exp_degree_6": ("    float p = c7;\n    p = fmaf(p, r, c6);", "    float p = c6;"),
    "exp_one_constant_reduction": ("    r = fmaf(-n, ln2_lo, r);", "    r = r;"),
    "bf16_truncate": ("    return (uint16_t)((u + 0x7fffu + lsb) >> 16);", "    return (uint16_t)((u + 0u * lsb) >> 16);"),
}


def build_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    tree = tmp_path / "oracle_copy"
    shutil.copytree(os.path.dirname(obuild.SRC), tree, ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    path = tree / "oracle.c"
    text = path.read_text()
    assert text.count(old) == 1, f"anchor for {name} not found exactly once"
    path.write_text(text.replace(old, new))
    lib = oracle.load(obuild.build(str(path), str(tree / "libmutant.so")))
    assert lib.oracle_source_sha256().decode() == hashlib.sha256(path.read_bytes()).hexdigest()
    return lib


def test_mutant_residual_before_act(tmp_path):
    lib = build_mutant(tmp_path, "residual_before_act")
    got = oracle.epilogue(np.array([[1.0]], np.float32), bias=np.array([-2.0], np.float32), act="relu",
                          residual=np.array([[-1.0]], np.float32), lib=lib)[0, 0]
    assert got != -1.0


@pytest.mark.parametrize("name", ["exp_degree_6", "exp_one_constant_reduction"])
def test_mutant_exp_breaks_accuracy(tmp_path, name):
    lib = build_mutant(tmp_path, name)
    xs = np.linspace(-87.0, 88.7, 20001, dtype=np.float32)
    worst = max(abs(oracle.ep_exp(float(x), lib=lib) - math.exp(float(x))) / ulp(math.exp(float(x))) for x in xs)
    assert worst > 2.0, worst


def test_mutant_bf16_truncate(tmp_path):
    lib = build_mutant(tmp_path, "bf16_truncate")
    v = np.array([[0x3f818000]], dtype=np.uint32).view(np.float32)
    assert int(oracle.epilogue(v, out="bf16", lib=lib)[0, 0]) != 0x3f82
