"""Bits independent of the number of compute units.

"Reproducible GPU inference", section "Three interventions, and what each was worth": the order contract
leaves nothing to the scheduler, so the number of multiprocessors, the tile schedule and the occupancy
cannot touch the bits. Here every kernel family runs on streams restricted to a subset of the compute
units (hipExtStreamCreateWithCUMask) and must give the bits of an unrestricted run, which in turn equal
the oracle's. The persistent tree GEMV sizes its grid from the device's CU count, so on a restricted
stream its workgroups queue behind one another; none of them waits on another, so the grid drains.

Each mask enables compute units in every one of the eight XCDs, whether the runtime deals mask bits to
the XCDs in blocks of 32 or round robin, so no XCD is left without a unit to run its workgroups."""
import ctypes as ct

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import dev_bf16, dev_f32, f32_bits, host_bits, say

pytestmark = pytest.mark.gpu

# 8 words = 256 compute units. Every word holds a set bit (one per XCD under a block deal of 32 bits) and
# the set bits cover every residue mod 8 (one per XCD under a round-robin deal).
MASKS = {
    "8cu": [1 << w for w in range(8)],
    "64cu": [0x000000FF] * 8,
    "128cu": [0x00FF00FF] * 8,
    "248cu": [0xFFFFFFFE] * 8,
}


def _hip_runtime():
    """The HIP runtime torch has loaded (the one the library binds to)."""
    import torch
    torch.cuda.init()
    with open("/proc/self/maps") as f:
        paths = sorted({ln.split()[-1] for ln in f if "libamdhip64.so" in ln})
    assert paths, "libamdhip64.so is not mapped"
    hip = ct.CDLL(paths[0])
    hip.hipExtStreamCreateWithCUMask.argtypes = [ct.POINTER(ct.c_void_p), ct.c_uint32, ct.POINTER(ct.c_uint32)]
    hip.hipExtStreamCreateWithCUMask.restype = ct.c_int
    hip.hipStreamDestroy.argtypes = [ct.c_void_p]
    hip.hipStreamDestroy.restype = ct.c_int
    hip.hipStreamSynchronize.argtypes = [ct.c_void_p]
    hip.hipStreamSynchronize.restype = ct.c_int
    return hip


@pytest.fixture(scope="module")
def g():
    import gemv_gemm_ordered_amd as g
    return g


@pytest.fixture(scope="module")
def streams():
    import torch
    props = torch.cuda.get_device_properties(0)
    assert props.multi_processor_count == 256, props.multi_processor_count
    hip = _hip_runtime()
    out = {}
    for name, words in MASKS.items():
        s = ct.c_void_p()
        arr = (ct.c_uint32 * len(words))(*words)
        rc = hip.hipExtStreamCreateWithCUMask(ct.byref(s), len(words), arr)
        assert rc == 0 and s.value, (name, rc)
        out[name] = torch.cuda.ExternalStream(s.value)
    yield out
    torch.cuda.synchronize()
    for st in out.values():
        hip.hipStreamSynchronize(st.cuda_stream)
        hip.hipStreamDestroy(st.cuda_stream)


def run_on(stream, fn):
    """fn(stream) after all work so far, then wait for it; returns fn's result."""
    import torch
    torch.cuda.synchronize()
    out = fn(stream)
    if stream is not None:
        stream.synchronize()
    torch.cuda.synchronize()
    return out


def check_everywhere(streams, fn, ref, what):
    """fn(stream) -> tensor: bits equal `ref` unrestricted and on every masked stream."""
    base = host_bits(run_on(None, fn))
    assert np.array_equal(base, ref), (what, "unrestricted")
    for name, st in streams.items():
        say(f"cu mask {name}: {what}")
        got = host_bits(run_on(st, fn))
        assert np.array_equal(got, ref), (what, name, int(np.count_nonzero(got != ref)))


def test_ordered_gemm(g, streams):
    A, W = synth.mlp_up(2, 256)
    ref = f32_bits(oracle.gemm_ordered(A, W, threads=16))
    dA, dW = dev_bf16(A), dev_bf16(W)
    check_everywhere(streams, lambda s: g.gemm_ordered(dA, dW, stream=s), ref, "gemm_ordered mlp M=256")
    Ag, Wg = synth.gpt2_projection(2, 64)
    refg = f32_bits(oracle.gemm_ordered(Ag, Wg))
    dAg, dWg = dev_bf16(Ag), dev_bf16(Wg)
    check_everywhere(streams, lambda s: g.gemm_ordered(dAg, dWg, stream=s), refg, "gemm_ordered gpt2 M=64")


def test_ordered_gemv_and_value_product(g, streams):
    import torch
    x, W, _ = synth.decode_gemv(2, 8)
    ref = f32_bits(oracle.gemm_ordered(x, W, threads=16))
    dx, dW = dev_bf16(x), dev_bf16(W)
    for M in (1, 8):
        check_everywhere(streams, lambda s: g.gemv_ordered(dx[:M], dW, stream=s), ref[:M], f"gemv_ordered M={M}")
    P, V = synth.pv_sequence(2, 0, 64, heads=4)
    refp = np.stack([f32_bits(oracle.gemm_ordered(P[h], V[h])) for h in range(4)])
    dP, dV = dev_f32(P), dev_bf16(V)

    def pv(s):
        O = torch.empty((4, 64, 128), device="cuda")
        g.gemm_ordered_grouped([(dP, dV, O)], stream=s)
        return O
    check_everywhere(streams, pv, refp, "value product L=64")


def test_tree_gemv_both_forms(g, streams):
    x, W, _ = synth.decode_gemv(2, 8)
    WT = np.ascontiguousarray(W.T)
    ref = f32_bits(oracle.gemv_tree(x, WT, threads=16))
    dx, dWT = dev_bf16(x), dev_bf16(WT)
    for M in (1, 4, 8):
        check_everywhere(streams, lambda s: g.gemv_tree(dx[:M], dWT, stream=s), ref[:M], f"gemv_tree M={M}")
        check_everywhere(streams, lambda s: g.test_gemv_instance("tree", 8, 2, dx[:M], dWT, stream=s), ref[:M],
                         f"gemv_tree one-group form M={M}")


def test_matrix_core_gemm_and_gemv(g, streams):
    A, W = synth.mlp_up(2, 512)
    ref = host_bits(g.gemm_mfma_invariant(dev_bf16(A), dev_bf16(W)))
    # sampled rows against the CPU bit model of the instruction
    rows = [0, 255, 511]
    assert np.array_equal(ref[rows], f32_bits(oracle.gemm_mfma(A[rows], W, threads=16)))
    dA, dW = dev_bf16(A), dev_bf16(W)
    check_everywhere(streams, lambda s: g.gemm_mfma_invariant(dA, dW, stream=s), ref, "gemm_mfma_invariant M=512")
    check_everywhere(streams, lambda s: g.test_gemm_mfma_tile128(dA, dW, stream=s), ref, "gemm_mfma 128x128 tile")
    dWT = dev_bf16(np.ascontiguousarray(W.T))
    for M in (1, 8):
        check_everywhere(streams, lambda s: g.gemv_mfma_invariant(dA[:M], dWT, stream=s), ref[:M],
                         f"gemv_mfma_invariant M={M}")
