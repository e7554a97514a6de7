"""The certificate engine (ggo_cert_*) on the host: its verdicts against the definition of the float
Freivalds check ("Same Bits on the CPU and the GPU", section "The CPU as a checker"), the escape law
of a cancelling fault under t independent sign vectors, back pressure on a small ring and the failure
log. No GPU: the engine is created in host mode and fed host rows."""
import numpy as np
import pytest

import oracle
import synth


@pytest.fixture(scope="module")
def g():
    import gemv_gemm_ordered_amd as g
    return g


@pytest.fixture(scope="module")
def data():
    x, W, _ = synth.decode_gemv(4, m_max=8, k=512, n=768)
    y = oracle.gemm_ordered(x, W)
    return x, W, y


def signs(seed, t, n):
    return np.stack([synth.rademacher(seed + v, "cert.r", n) for v in range(t)])


def test_honest_rows_pass_and_single_faults_are_caught(g, data):
    x, W, y = data
    eng = g.CertEngine(512, 768, slots=4, workers=2, host_only=True)
    mid = eng.add_matrix(W, signs(1, 1, 768))
    for m in range(8):
        eng.submit_host(mid, x[m], y[m], token=m)
    for m in range(8):                       # a planted +0.005 on one output of every row
        yb = y[m].copy()
        yb[37 * m + 5] += np.float32(0.005)
        eng.submit_host(mid, x[m], yb, token=100 + m)
    st = eng.drain()
    assert st["submitted"] == st["checked"] == 16 and st["failed"] == 8 and not st["copy_error"]
    assert sorted(t for t, _ in eng.failures()) == list(range(100, 108))
    assert 0 < st["max_honest_ratio"] < 0.125
    eng.close()


def test_verdicts_match_freivalds_check(g, data):
    x, W, y = data
    r = signs(2, 3, 768)
    eng = g.CertEngine(512, 768, slots=8, workers=3, host_only=True)
    mid = eng.add_matrix(W, r)
    rng = np.random.default_rng(0)
    expect = []
    for i in range(40):
        m = i % 8
        yb = y[m].copy()
        if rng.random() < 0.5:
            yb[rng.integers(0, 768)] += np.float32(rng.choice([0.005, -0.003, 1e-6]))
        eng.submit_host(mid, x[m], yb, token=i)
        ok = all(oracle.freivalds_check(oracle.freivalds_prepare(W, r[v]), r[v], x[m], yb)[0] for v in range(3))
        expect.append(ok)
    eng.drain()
    failed = sorted(t for t, _ in eng.failures())
    assert failed == [i for i, ok in enumerate(expect) if not ok]
    eng.close()


def test_cancelling_pair_escapes_iff_every_sign_vector_agrees(g, data):
    # +d at j1 and -d at j2 changes r.y by d (r[j1] - r[j2]): zero exactly when r[j1] == r[j2]. With t
    # independent vectors the pair escapes iff all t agree on it: probability 2^-t over random pairs.
    x, W, y = data
    rng = np.random.default_rng(5)
    pairs = [tuple(rng.choice(768, 2, replace=False)) for _ in range(400)]
    for t in (1, 2, 4):
        r = signs(10 * t, t, 768)
        eng = g.CertEngine(512, 768, slots=16, workers=4, host_only=True)
        mid = eng.add_matrix(W, r)
        for i, (j1, j2) in enumerate(pairs):
            yb = y[0].copy()
            yb[j1] += np.float32(0.05)
            yb[j2] -= np.float32(0.05)
            eng.submit_host(mid, x[0], yb, token=i)
        eng.drain()
        caught = {tok for tok, _ in eng.failures()}
        escaped = [i for i in range(len(pairs)) if i not in caught]
        want = [i for i, (j1, j2) in enumerate(pairs) if all(r[v, j1] == r[v, j2] for v in range(t))]
        assert escaped == want, t
        assert abs(len(escaped) / len(pairs) - 2.0 ** -t) < 4 * (2.0 ** -t * (1 - 2.0 ** -t) / len(pairs)) ** 0.5, t
        eng.close()


def test_transposed_weight_gives_the_same_verdicts(g, data):
    x, W, y = data
    r = signs(3, 2, 768)
    a = g.CertEngine(512, 768, slots=4, workers=1, host_only=True)
    b = g.CertEngine(512, 768, slots=4, workers=1, host_only=True)
    ma, mb = a.add_matrix(W, r), b.add_matrix(np.ascontiguousarray(W.T), r, transposed=True)
    for m in range(8):
        yb = y[m].copy()
        yb[m] += np.float32(0.004 * (m % 2))
        a.submit_host(ma, x[m], yb, m)
        b.submit_host(mb, x[m], yb, m)
    a.drain(), b.drain()
    assert a.failures() == b.failures() and len(a.failures()) == 4
    a.close(), b.close()


def test_small_ring_back_pressure(g, data):
    x, W, y = data
    eng = g.CertEngine(512, 768, slots=2, workers=1, host_only=True)
    mid = eng.add_matrix(W, signs(7, 1, 768))
    for i in range(200):
        eng.submit_host(mid, x[i % 8], y[i % 8], token=i)
    st = eng.drain()
    assert st["submitted"] == st["checked"] == 200 and st["failed"] == 0
    eng.close()


def test_bad_arguments(g, data):
    x, W, y = data
    with pytest.raises(g.GGOError):
        g.CertEngine(0, 10, host_only=True)
    eng = g.CertEngine(512, 768, slots=2, workers=1, host_only=True)
    with pytest.raises(g.GGOError):
        eng.add_matrix(W, np.zeros((1, 768), np.int8))           # signs must be +-1
    with pytest.raises(g.GGOError):
        eng.add_matrix(np.zeros((1024, 768), np.uint16), signs(1, 1, 768))   # K above max_K
    eng.close()


def test_matrices_added_while_checks_run(g, data):
    """Matrices registered while other rows are being checked: every earlier matrix stays valid (entries
    never move), every row is checked against its own matrix, and an unknown id is refused."""
    import threading
    x, W, y = data
    eng = g.CertEngine(512, 768, slots=4, workers=3, host_only=True)
    mid0 = eng.add_matrix(W, signs(11, 1, 768))
    added = []

    def adder():
        for i in range(40):
            added.append(eng.add_matrix(W, signs(20 + i, 1, 768)))

    th = threading.Thread(target=adder)
    th.start()
    for i in range(300):
        eng.submit_host(mid0 if i % 3 or not added else added[-1], x[i % 8], y[i % 8], token=i)
    th.join()
    for mid in added:
        eng.submit_host(mid, x[mid % 8], y[mid % 8], token=1000 + mid)
    st = eng.drain()
    assert added == list(range(1, 41))
    assert st["checked"] == 340 and st["failed"] == 0
    xr, yr = np.ascontiguousarray(x[0]), np.ascontiguousarray(y[0])
    assert g.lib.ggo_cert_submit_host(eng.h, 41, xr.ctypes.data, yr.ctypes.data, 0) == -1
    eng.close()
