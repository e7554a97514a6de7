"""Seeded synthetic inputs for the batch-invariant matmul library.

This module is shared by the tests, the benchmark and the smoke check, and it
serves both the CPU oracle and the GPU path. It holds none of the matmul
arithmetic: it only draws numbers and rounds them to the storage formats.

Generator (one definition, counter based, so any element or row can be
regenerated on its own):

* ``splitmix64`` (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014) applied to ``stream_key + (i + 1) * golden_gamma``
  gives 64 random bits for counter ``i``.
* A uniform in [0, 1) is the top 53 bits times 2**-53.
* A standard normal for element ``i`` is the Box-Muller cosine branch over the
  uniforms of counters ``2i`` and ``2i + 1``, evaluated in float64.
* Values are scaled by sigma in float64, rounded to float32 (round to nearest
  even), then to bfloat16 (round to nearest even on bit 16).

Each tensor of a workload has its own stream key derived from ``(seed, tag)``,
so the content of row ``m`` of an ``[M, K]`` operand is the same for every
``M``: element ``(m, k)`` always uses counter ``m * K + k``.
"""
from __future__ import annotations

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)
_TWO_PI = 2.0 * np.pi


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _MIX1
    z = (z ^ (z >> np.uint64(27))) * _MIX2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, tag: str) -> int:
    """64-bit key of the stream named ``tag`` under ``seed`` (FNV-1a of the tag, mixed)."""
    h = 0xCBF29CE484222325
    for ch in tag.encode():
        h = ((h ^ ch) * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    with np.errstate(over="ignore"):
        z = np.array([(h ^ (seed * 0x9E3779B97F4A7C15)) & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64)
        return int(_mix(z)[0])


def bits64(key: int, start: int, count: int) -> np.ndarray:
    """splitmix64 outputs for counters ``start .. start+count-1`` of stream ``key``."""
    with np.errstate(over="ignore"):
        i = np.arange(start, start + count, dtype=np.uint64)
        z = np.uint64(key) + (i + np.uint64(1)) * _GAMMA
        return _mix(z)


def uniform01(key: int, start: int, count: int) -> np.ndarray:
    return (bits64(key, start, count) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal_f64(key: int, start: int, count: int) -> np.ndarray:
    """Standard normals for elements ``start .. start+count-1`` (float64)."""
    u = uniform01(key, 2 * start, 2 * count)
    u1 = 1.0 - u[0::2]          # in (0, 1]
    u2 = u[1::2]
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(_TWO_PI * u2)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest even; returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, tag: str, shape, sigma: float = 1.0, chunk: int = 1 << 22) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of sigma * N(0, 1), shape ``shape``, row-major counters."""
    n = int(np.prod(shape))
    key = stream_key(seed, tag)
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        c = min(chunk, n - s)
        v = (normal_f64(key, s, c) * sigma).astype(np.float32)
        out[s:s + c] = f32_to_bf16_bits(v)
    return out.reshape(shape)


def normal_f32(seed: int, tag: str, shape, sigma: float = 1.0, chunk: int = 1 << 22) -> np.ndarray:
    n = int(np.prod(shape))
    key = stream_key(seed, tag)
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, chunk):
        c = min(chunk, n - s)
        out[s:s + c] = (normal_f64(key, s, c) * sigma).astype(np.float32)
    return out.reshape(shape)


def rademacher(seed: int, tag: str, n: int) -> np.ndarray:
    """int8 vector of +1/-1 (the sign is the top bit of each 64-bit draw)."""
    b = bits64(stream_key(seed, tag), 0, n) >> np.uint64(63)
    return (1 - 2 * b.astype(np.int64)).astype(np.int8)


def softmax_rows_f32(seed: int, tag: str, rows: int, cols: int, row_start: int = 0) -> np.ndarray:
    """Rows of softmax(N(0,1) float32 logits): each row is computed in float64 and rounded to float32.

    Row ``i`` (absolute index ``row_start + i``) uses counters ``(row_start+i)*cols ..``, so any
    row block can be generated on its own.
    """
    key = stream_key(seed, tag)
    logits = normal_f64(key, row_start * cols, rows * cols).astype(np.float32).astype(np.float64)
    logits = logits.reshape(rows, cols)
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def integer_bf16(seed: int, tag: str, shape, lo: int = -4, hi: int = 4) -> np.ndarray:
    """bfloat16 bit patterns of integers uniform in [lo, hi] (exact in bfloat16)."""
    n = int(np.prod(shape))
    span = hi - lo + 1
    v = (bits64(stream_key(seed, tag), 0, n) % np.uint64(span)).astype(np.int64) + lo
    return f32_to_bf16_bits(v.astype(np.float32)).reshape(shape)


# ---------------------------------------------------------------------------
# The workloads: shapes and distributions of the five configurations.
# ---------------------------------------------------------------------------

def gpt2_projection(seed: int, m_max: int = 512):
    """A[m_max, 768] ~ N(0,1), W[768, 768] ~ N(0, 0.02) (bf16 bits). Smaller M are row prefixes."""
    A = normal_bf16(seed, "gpt2.A", (m_max, 768), 1.0)
    W = normal_bf16(seed, "gpt2.W", (768, 768), 0.02)
    return A, W


def decode_gemv(seed: int, m_max: int = 8, k: int = 4096, n: int = 4096):
    """x[m_max, 4096] ~ N(0,1), W[4096, 4096] ~ N(0, 0.02), r in {+-1}^4096."""
    x = normal_bf16(seed, "gemv.x", (m_max, k), 1.0)
    W = normal_bf16(seed, "gemv.W", (k, n), 0.02)
    r = rademacher(seed, "gemv.r", n)
    return x, W, r


def mlp_up(seed: int, m_max: int = 2048):
    """A[m_max, 1024] ~ N(0,1), W[1024, 4096] ~ N(0, 0.02)."""
    A = normal_bf16(seed, "mlp.A", (m_max, 1024), 1.0)
    W = normal_bf16(seed, "mlp.W", (1024, 4096), 0.02)
    return A, W


def proj_7b(seed: int, n: int = 4096, m: int = 4096, k: int = 4096):
    """A[4096, 4096] ~ N(0,1), W[4096, n] ~ N(0, 0.02) with n in {4096, 11008}."""
    A = normal_bf16(seed, "7b.A", (m, k), 1.0)
    W = normal_bf16(seed, f"7b.W{n}", (k, n), 0.02)
    return A, W


def pv_sequence(seed: int, seq_id: int, L: int, heads: int = 32, d: int = 128):
    """One sequence of the value product: P[heads, L, L] fp32 softmax rows, V[heads, L, d] bf16."""
    P = np.empty((heads, L, L), dtype=np.float32)
    for h in range(heads):
        P[h] = softmax_rows_f32(seed, f"pv.P.{seq_id}.{h}.{L}", L, L)
    V = normal_bf16(seed, f"pv.V.{seq_id}.{L}", (heads, L, d), 1.0)
    return P, V


PV_LENGTHS = (1, 15, 16, 64, 256, 1024, 5000)
