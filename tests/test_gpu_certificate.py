"""The Freivalds certificate over real GPU GEMV outputs (decode shape): honest
rows pass with the frozen constant, a planted +0.005 or +0.05 on one output is
caught ("Same Bits on the CPU and the GPU", section "The CPU as a checker")."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import dev_bf16

pytestmark = pytest.mark.gpu


def test_gpu_gemv_certified(tmp_path):
    import gemv_gemm_ordered_amd as g
    import torch
    x, W, r = synth.decode_gemv(0, 8)
    y = g.gemv_ordered(dev_bf16(x), dev_bf16(W))
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    f = g.freivalds_prepare(W, synth.stream_key(0, "gemv.r"))
    assert np.array_equal(f.signs(), r)
    j = int(synth.bits64(synth.stream_key(0, "fault.j"), 0, 1)[0] % 4096)
    oprep = oracle.freivalds_prepare(W, r)
    for m in range(8):
        ok, rho, sigma, tau, bound = f.check(x[m], yh[m])
        assert ok and rho <= bound, (m, rho, tau)
        assert oracle.freivalds_check(oprep, r, x[m], yh[m])[0]
        for delta in (0.005, 0.05):
            yb = yh[m].copy()
            yb[j] += np.float32(delta)
            assert not f.check(x[m], yb)[0]
            assert not oracle.freivalds_check(oprep, r, x[m], yb)[0]
