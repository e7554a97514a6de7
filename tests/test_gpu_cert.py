"""The certificate engine in a decode loop on the GPU: every output row of every matrix of every token is
copied asynchronously (engine stream, after the GEMV on the caller's stream) and checked on host
threads; faults planted on the device outputs of chosen tokens are exactly the failures reported."""
import numpy as np
import pytest

import synth
from tests.gpu_util import dev_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import gemv_gemm_ordered_amd as g
    return g


def test_decode_loop_catches_exactly_the_planted_faults(g):
    import torch
    shapes = [(4096, 4096), (11008, 4096), (4096, 11008)]   # (N, K) of W^T
    WTs = [synth.normal_bf16(1 + i, "cert.WT", (n, k), 0.02) for i, (n, k) in enumerate(shapes)]
    eng = g.CertEngine(11008, 11008, slots=32, workers=4)
    mids = [eng.add_matrix(wt, np.stack([synth.rademacher(9 + i, "cert.r", wt.shape[0]) for i in range(2)]),
                           transposed=True) for wt in WTs]
    dW = [dev_bf16(wt) for wt in WTs]
    keep, planted = [], set()
    rng = np.random.default_rng(1)
    say("cert decode loop: 24 tokens x 3 matrices")
    for tok in range(24):
        for i, (n, k) in enumerate(shapes):
            x = dev_bf16(synth.normal_bf16(100 * tok + i, "cert.x", (1, k)))
            y = g.gemv_tree(x, dW[i])
            if tok % 5 == 3 and i == tok % 3:
                # +0.05: above the detection floor tau = c_f * 2^-24 sqrt(K) sum_k |x_k| ||W[k,:]||_2 of
                # every matrix here (about 0.009 at K = 11008, 0.002 at K = 4096)
                y[0, int(rng.integers(0, n))] += 0.05
                planted.add((tok, mids[i]))
            eng.submit(mids[i], x[0], y[0], token=tok)
            keep.append((x, y))                  # the rows must outlive their copies
    st = eng.drain()
    torch.cuda.synchronize()
    assert st["submitted"] == st["checked"] == 72 and not st["copy_error"]
    assert set(eng.failures()) == planted and st["failed"] == len(planted)
    assert 0 < st["max_honest_ratio"] < 0.125
    eng.close()


def test_batched_rows_catch_exactly_the_planted_faults(g):
    import torch
    shapes = [(4096, 4096), (11008, 4096), (4096, 11008)]
    WTs = [synth.normal_bf16(7 + i, "certb.WT", (n, k), 0.02) for i, (n, k) in enumerate(shapes)]
    eng = g.CertEngine(11008, 11008, slots=16, workers=3)
    mids = [eng.add_matrix(wt, synth.rademacher(30 + i, "certb.r", wt.shape[0])[None, :], transposed=True)
            for i, wt in enumerate(WTs)]
    dW = [dev_bf16(wt) for wt in WTs]
    keep, planted = [], set()
    say("cert batched rows: 30 tokens x 3 matrices")
    for tok in range(30):
        xs, ys = [], []
        for i, (n, k) in enumerate(shapes):
            x = dev_bf16(synth.normal_bf16(1000 + 7 * tok + i, "certb.x", (1, k)))
            y = g.gemv_tree(x, dW[i])
            if tok % 4 == 1 and i == (tok // 4) % 3:
                y[0, (97 * tok) % n] -= 0.05
                planted.add((tok, mids[i]))
            xs.append(x[0])
            ys.append(y[0])
        eng.submit_rows(mids, xs, ys, token=tok)
        keep.append((xs, ys))
    st = eng.drain()
    torch.cuda.synchronize()
    assert st["submitted"] == st["checked"] == 90 and not st["copy_error"]
    assert set(eng.failures()) == planted
    eng.close()


def test_batched_rows_at_unaligned_addresses(g):
    """Rows that start off a 16-byte boundary (inside a padded buffer) take the gather's 2-byte copies; the
    rest take 16-byte copies. Honest rows pass and a planted fault is caught either way."""
    import torch
    shapes = [(4096, 4096), (11008, 4096), (4096, 11008), (1000, 1004)]
    WTs = [synth.normal_bf16(50 + i, "certu.WT", (n, k), 0.02) for i, (n, k) in enumerate(shapes)]
    eng = g.CertEngine(11008, 11008, slots=16, workers=2)
    mids = [eng.add_matrix(wt, synth.rademacher(60 + i, "certu.r", wt.shape[0])[None, :], transposed=True)
            for i, wt in enumerate(WTs)]
    dW = [dev_bf16(wt) for wt in WTs]
    keep, planted = [], set()
    say("cert batched rows at unaligned addresses: 6 tokens x 4 matrices")
    for tok in range(6):
        xs, ys = [], []
        for i, (n, k) in enumerate(shapes):
            shift = (tok + i) % 3                      # 0: aligned; 1, 2: x and y off 16-byte boundaries
            xb = torch.zeros((1, k + 8), dtype=torch.bfloat16, device="cuda")
            xb[0, shift:shift + k] = dev_bf16(synth.normal_bf16(200 + 7 * tok + i, "certu.x", (1, k)))[0]
            x = xb[0, shift:shift + k]
            yb = torch.zeros((n + 8,), device="cuda")
            y = yb[shift:shift + n]
            g.gemv_tree(x[None, :].contiguous(), dW[i], y=y[None, :])
            if i == 1 and tok in (2, 4):                # shift 0 at token 2, shift 2 at token 4
                y[(31 * tok) % n] += 0.05
                planted.add((tok, mids[i]))
            xs.append(x)
            ys.append(y)
        eng.submit_rows(mids, xs, ys, token=tok)
        keep.append((xs, ys))
    st = eng.drain()
    torch.cuda.synchronize()
    assert st["submitted"] == st["checked"] == 24 and not st["copy_error"]
    assert set(eng.failures()) == planted and len(planted) == 2
    eng.close()


def test_late_copy_takes_the_stream_path(g):
    """A row whose copy waits behind a long kernel on the caller's stream (an ordered 4096^3 GEMM, a few
    ms) arrives after the workers' 2 ms of polling: the worker then synchronises the engine's stream and
    still checks the row."""
    import torch
    K = N = 4096
    WT = synth.normal_bf16(3, "certl.WT", (N, K), 0.02)
    eng = g.CertEngine(K, N, slots=4, workers=1)
    mid = eng.add_matrix(WT, synth.rademacher(5, "certl.r", N)[None, :], transposed=True)
    x = dev_bf16(synth.normal_bf16(4, "certl.x", (1, K)))
    y = g.gemv_tree(x, dev_bf16(WT))
    A = dev_bf16(synth.normal_bf16(6, "certl.A", (4096, 4096)))
    B = dev_bf16(synth.normal_bf16(7, "certl.B", (4096, 4096), 0.02))
    torch.cuda.synchronize()
    say("cert late copy: a long GEMM ahead of the submit")
    C = g.gemm_ordered(A, B)                 # queued ahead of the copy on the same stream
    eng.submit(mid, x[0], y[0], token=0)
    st = eng.drain()
    torch.cuda.synchronize()
    assert st["checked"] == 1 and st["failed"] == 0 and not st["copy_error"]
    assert st["wait_seconds"] > 0.002, st
    eng.close()
    del C


def test_batch_larger_than_the_ring_is_refused(g):
    """A batch holds its slots until all are taken, so one larger than the ring could never be served: the
    call must return an error at once instead of waiting forever."""
    import torch
    WT = synth.normal_bf16(3, "certr.WT", (64, 128), 0.02)
    eng = g.CertEngine(128, 64, slots=2, workers=1)
    mid = eng.add_matrix(WT, synth.rademacher(3, "certr.r", 64)[None, :], transposed=True)
    x = dev_bf16(synth.normal_bf16(3, "certr.x", (3, 128)))
    y = g.gemv_tree(x, dev_bf16(WT))
    with pytest.raises(g.GGOError):
        eng.submit_rows([mid] * 3, [x[i] for i in range(3)], [y[i] for i in range(3)], token=0)
    eng.submit_rows([mid] * 2, [x[i] for i in range(2)], [y[i] for i in range(2)], token=1)
    st = eng.drain()
    torch.cuda.synchronize()
    assert st["submitted"] == st["checked"] == 2 and st["failed"] == 0 and not st["copy_error"]
    eng.close()
