#!/usr/bin/env python3
"""Benchmark of the batch-invariant matmul library on one MI355X.

Headline workload (one "step"): the decode GEMV of x[M, 4096] (bf16) by a
4096 x 4096 bf16 weight, binary32 result, for M = 1, 4 and 8, through
gemv_tree (the tree order; the weight stored as a linear layer stores it,
[N, K] with k contiguous). Sixteen copies of the weight (512 MiB, twice the
256 MB Infinity Cache) are rotated so every launch streams its weight from
HBM. The value is GB/s of algorithmic traffic (2KN + 2MK + 4MN bytes per
launch) over the timed steps. The timed steps are captured once in a HIP graph
and replayed, so host launch overhead is not timed; HIP events on the launch
stream bracket the replay.

Beside it, in the same JSON line:
  roofline      the tree GEMV kernel against 8 TB/s HBM
  cpu_baseline  the CPU oracle of the same step, one core, for ~10 s
  per_M         per-M time of gemv_tree, of gemv_ordered (the one-lane chain
                contract, weight [K, N]) and of torch.mm (hipBLASLt, not batch
                invariant) on the same data
  certificate   Freivalds checks of sampled rows (honest pass, planted fault caught)
  paths         the other paths at their workloads: ordered GEMM and MFMA GEMM
                TFLOP/s (MLP up-projection, 7B projections), the value product,
                the fused epilogue against the same steps as separate kernels,
                and torch.matmul (hipBLASLt, not batch invariant) on the same shapes
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2516.0          # 256 CU x 4096 flop/clk x 2.4 GHz, dense
# The order contract multiplies and adds separately (two binary32 ops per MAC,
# packed binary32 disabled). gfx950 executes a wave64 binary32 VALU op in two
# passes of 32 lanes (measured: a SIMD completes one about every 2.2-2.5 clocks
# with two waves), so 256 CU x 4 SIMD x 32 lanes x 2.4 GHz = 78.6 T ops/s, i.e.
# 78.6 TFLOP/s counting 2 flop per MAC -- half the 157.3 TFLOP/s nominal (FMA).
VALU_CONTRACT_PEAK_TFS = 78.6
VALU_NOMINAL_PEAK_TFS = 157.3


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def dev_bf16(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def time_region(fn, reps: int, warmup: int = 2) -> float:
    """Mean ms per call of fn(), HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / reps


def graph_time(fn, reps: int) -> float:
    """Mean ms per call of fn(i) for i = 0 .. reps-1, captured once in a HIP graph and replayed
    (HIP events on the current stream), so host launch overhead is not timed."""
    import torch
    for i in range(2):
        fn(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(reps):
            fn(i)
    graph.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    graph.replay()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / reps


def gemv_bytes(M, K=4096, N=4096):
    return 2 * K * N + 2 * M * K + 4 * M * N


# Host threads for the all-cores legs: the CPU share of one GPU on the MI355X boxes is 16 cores, whatever
# nproc reports there, so the leg uses at most that many (nproc and the affinity mask are recorded beside it).
HOST_SHARE_THREADS = 16


def _host_threads():
    return max(1, min(HOST_SHARE_THREADS, len(os.sched_getaffinity(0))))


class _one_core:
    """Pin the calling thread (where a threads=1 oracle call runs) to one core of its mask, then restore."""

    def __enter__(self):
        self.mask = os.sched_getaffinity(0)
        self.core = min(self.mask)
        os.sched_setaffinity(0, {self.core})
        return self

    def __exit__(self, *exc):
        os.sched_setaffinity(0, self.mask)


def _repeat(fn, seconds):
    """Calls of fn() until `seconds` pass; returns (calls, elapsed)."""
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            return n, dt


def cpu_baseline(x, WT, ms, seconds):
    """The oracle of the headline step (oracle.gemv_tree): one core (pinned), whole steps until `seconds`
    pass, then over the host threads for half as long."""
    import oracle
    with _one_core() as pin:
        steps, dt = _repeat(lambda: [oracle.gemv_tree(x[:M], WT, threads=1) for M in ms], seconds)
    gbs = steps * sum(gemv_bytes(M) for M in ms) / dt / 1e9
    threads = _host_threads()
    steps_all, dt_all = _repeat(lambda: [oracle.gemv_tree(x[:M], WT, threads=threads) for M in ms], seconds / 2)
    gbs_all = steps_all * sum(gemv_bytes(M) for M in ms) / dt_all / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} full decode steps (M={','.join(map(str, ms))}, K=N=4096) of the tree-order "
                      f"oracle, plain C, single-threaded, pinned to core {pin.core}, {dt:.1f} s",
            "all_cores": {"value": round(gbs_all, 4), "cores": threads,
                          "sample": f"{steps_all} steps, outputs split over {threads} threads (the CPU share of "
                                    f"one GPU), {dt_all:.1f} s"},
            "cpu_model": cpu_model(), "nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}


def cpu_oracle_configs(seconds=1.0):
    """The oracle on every workload of the path, one core (pinned) and over the host threads: a stated
    sample of each (whole outputs; rows are independent, so a row subset scales linearly), repeated for
    about `seconds`, as GFLOP/s of algorithmic work and the time the whole workload would take."""
    import oracle
    import synth
    threads = _host_threads()
    out = {}

    def leg(name, path, fn_one, fn_all, flop, sample, full_flop, flop_all=None):
        with _one_core():
            n1, t1 = _repeat(fn_one, seconds)
        na, ta = _repeat(fn_all, seconds / 2)
        g1, ga = n1 * flop / t1 / 1e9, na * (flop_all or flop) / ta / 1e9
        out[name] = {"oracle": path, "gflops_1core": round(g1, 4), "gflops_all_cores": round(ga, 4),
                     "threads": threads, "sample": sample,
                     "full_workload_s_1core": round(full_flop / (g1 * 1e9), 2),
                     "full_workload_s_all_cores": round(full_flop / (ga * 1e9), 2)}

    A, W = synth.gpt2_projection(0, 512)
    f = 2.0 * 512 * 768 * 768
    leg("gpt2_proj_M512_N768_K768", "gemm_ordered", lambda: oracle.gemm_ordered(A, W),
        lambda: oracle.gemm_ordered(A, W, threads=threads), f, "all 512 rows", f)
    x, Wd, _ = synth.decode_gemv(0, 8)
    f = 2.0 * 8 * 4096 * 4096
    leg("decode_M8_N4096_K4096", "gemm_ordered (one-lane chain)", lambda: oracle.gemm_ordered(x, Wd),
        lambda: oracle.gemm_ordered(x, Wd, threads=8), f, "all 8 rows (at most 8 threads: one per row)", f)
    A = synth.normal_bf16(0, "mlp.A", (256, 1024), 1.0)
    W = synth.normal_bf16(0, "mlp.W", (1024, 4096), 0.02)
    leg("mlp_up_M2048_N4096_K1024", "gemm_ordered", lambda: oracle.gemm_ordered(A, W),
        lambda: oracle.gemm_ordered(A, W, threads=threads), 2.0 * 256 * 4096 * 1024,
        "rows 0-255 of 2048, scaled", 2.0 * 2048 * 4096 * 1024)
    leg("mlp_up_M2048_N4096_K1024_mfma_model", "gemm_mfma (bit model of the matrix-core GEMM)",
        lambda: oracle.gemm_mfma(A[:2], W), lambda: oracle.gemm_mfma(A[:2 * threads], W, threads=threads),
        2.0 * 2 * 4096 * 1024, f"rows 0-1 of 2048 on one core, rows 0-{2 * threads - 1} over the threads, scaled",
        2.0 * 2048 * 4096 * 1024, flop_all=2.0 * 2 * threads * 4096 * 1024)
    A = synth.normal_bf16(0, "7b.A", (32, 4096), 1.0)
    W = synth.normal_bf16(0, "7b.W4096", (4096, 4096), 0.02)
    leg("7b_qkvo_M4096_N4096_K4096", "gemm_ordered", lambda: oracle.gemm_ordered(A, W),
        lambda: oracle.gemm_ordered(A, W, threads=threads), 2.0 * 32 * 4096 * 4096,
        "rows 0-31 of 4096, scaled", 2.0 * 4096 ** 3)
    P = synth.softmax_rows_f32(0, "pv.P.0.0.5000", 256, 5000)
    V = synth.normal_bf16(0, "pv.V.0.5000", (5000, 128), 1.0)
    leg("pv_L5000_h32_d128", "gemm_ordered (binary32 P)", lambda: oracle.gemm_ordered(P, V),
        lambda: oracle.gemm_ordered(P, V, threads=threads), 2.0 * 256 * 5000 * 128,
        "query rows 0-255 of head 0, scaled to 32 heads x 5000 rows", 2.0 * 32 * 5000 * 5000 * 128)
    return out


def cpu_model():
    """The host CPU's full model name as /proc/cpuinfo reports it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def certificate(g, x, W, r, ys, ms):
    import ctypes as ct
    import numpy as np
    import torch

    import synth
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    f = g.freivalds_prepare(W, synth.stream_key(0, "gemv.r"))   # the signs of the workload's r stream
    t_prep = time.perf_counter() - t0
    assert np.array_equal(f.signs(), r)
    y8 = ys[ms[-1]]
    t1 = time.perf_counter()
    yh = y8.cpu().numpy()
    t_d2h = (time.perf_counter() - t1) / y8.shape[0]
    checks, worst, t_check = 0, 0.0, 0.0
    for m in range(yh.shape[0]):
        t2 = time.perf_counter()
        ok, rho, sigma, tau, bound = f.check(x[m], yh[m])
        t_check += time.perf_counter() - t2
        checks += ok
        worst = max(worst, rho / sigma)
    j = 1234
    yb = yh[0].copy()
    yb[j] += np.float32(0.005)
    caught = not f.check(x[0], yb)[0]
    # the library's check itself: the C entry point called directly on host rows, 200 rows
    out = np.empty(4, dtype=np.float64)
    xr = [np.ascontiguousarray(x[m]) for m in range(yh.shape[0])]
    yr = [np.ascontiguousarray(yh[m], dtype=np.float32) for m in range(yh.shape[0])]
    calls = [(f.h, xr[m].ctypes.data, yr[m].ctypes.data, ct.c_double(0.125), out.ctypes.data)
             for m in range(yh.shape[0])]
    for c in calls:
        g.lib.freivalds_check(*c)
    reps = 200
    t3 = time.perf_counter()
    for i in range(reps):
        g.lib.freivalds_check(*calls[i % len(calls)])
    t_c = (time.perf_counter() - t3) / reps
    f.close()
    return {"honest_pass": f"{checks}/{yh.shape[0]}", "max_honest_ratio": round(worst, 5), "c_f": 0.125,
            "planted_0.005_caught": caught, "us_per_check": round(1e6 * t_c, 2),
            "us_per_check_through_python_binding": round(1e6 * t_check / yh.shape[0], 2),
            "d2h_us_per_row_pair": round(1e6 * t_d2h, 2), "prepare_ms": round(1e3 * t_prep, 2)}


def paths(g, reps):
    """Throughput of the other paths at their workloads (seeded torch data, timing only)."""
    import torch
    torch.manual_seed(0)
    out = {}

    def randn_bf16(shape, std):
        return (torch.randn(shape, device="cuda", dtype=torch.float32) * std).to(torch.bfloat16)

    def mm_blaslt(A, W):
        try:
            return torch.mm(A, W, out_dtype=torch.float32)
        except TypeError:
            return torch.mm(A, W)

    # GPT-2-small projection, A[M,768] x W[768,768]: launch- and latency-bound, reported as time per call.
    # gemv_ordered (M <= 16) gives gemm_ordered's bits with a decode-shaped kernel.
    W = randn_bf16((768, 768), 0.02)
    for M in (1, 8, 64):
        A = randn_bf16((M, 768), 1.0)
        rec = {}
        fns = [("ordered", lambda i: g.gemm_ordered(A, W)), ("mfma", lambda i: g.gemm_mfma_invariant(A, W)),
               ("hipblaslt", lambda i: mm_blaslt(A, W))]
        if M <= 16:
            fns.insert(1, ("gemv_ordered", lambda i: g.gemv_ordered(A, W)))
        for name, fn in fns:
            rec[f"{name}_us"] = round(1e3 * graph_time(fn, 32), 2)
        out[f"gpt2_proj_M{M}_N768_K768"] = rec
    del W, A

    # MLP up-projection and 7B projections: ordered VALU, MFMA invariant, hipBLASLt
    # (7b_up_shard8: one GPU's share of the up-projection's W split 8 ways along N)
    shapes = [("mlp_up", m, 4096, 1024) for m in (64, 128, 256, 512, 1024, 2048)] + [
              ("7b_qkvo", 4096, 4096, 4096), ("7b_up", 4096, 11008, 4096), ("7b_up_shard8", 4096, 1376, 4096)]
    for name, M, N, K in shapes:
        A = randn_bf16((M, K), 1.0)
        W = randn_bf16((K, N), 0.02)
        C = torch.empty((M, N), device="cuda")
        flop = 2.0 * M * N * K
        rec = {}
        # each leg captured in a HIP graph and replayed (no host launch overhead in the small shapes' times)
        gr = 8 if flop > 1e11 else 32
        if name == "mlp_up":
            t = graph_time(lambda i: g.gemm_ordered(A, W, C=C), max(2, gr // 4))
            rec["ordered_tflops"] = round(flop / t / 1e9, 2)
            rec["ordered_frac_contract_peak"] = round(flop / t / 1e9 / VALU_CONTRACT_PEAK_TFS, 4)
            rec["ordered_frac_nominal_peak"] = round(flop / t / 1e9 / VALU_NOMINAL_PEAK_TFS, 4)
        t = graph_time(lambda i: g.gemm_mfma_invariant(A, W, C=C), gr)
        rec["mfma_tflops"] = round(flop / t / 1e9, 1)
        rec["mfma_frac_peak"] = round(flop / t / 1e9 / MFMA_BF16_PEAK_TFS, 4)
        tb = graph_time(lambda i: mm_blaslt(A, W), gr)
        rec["hipblaslt_tflops"] = round(flop / tb / 1e9, 1)
        rec["mfma_vs_hipblaslt"] = round(tb / t, 3)
        out[f"{name}_M{M}_N{N}_K{K}"] = rec
        del A, W, C
    # invariance control on the MLP shape: row 0's bits at each M against M = 2048, for the MFMA path and
    # for hipBLASLt (the control: if its rows never moved, the invariance shown here would be trivial)
    A = randn_bf16((2048, 1024), 1.0)
    W = randn_bf16((1024, 4096), 0.02)
    ref_m = g.gemm_mfma_invariant(A, W)[0].view(torch.int32).clone()
    ref_b = mm_blaslt(A, W)[0].float().view(torch.int32).clone()
    moved_m, moved_b = [], []
    for M in (1, 2, 8, 64, 128, 256, 512, 1024):
        if not torch.equal(g.gemm_mfma_invariant(A[:M], W)[0].view(torch.int32), ref_m):
            moved_m.append(M)
        if not torch.equal(mm_blaslt(A[:M], W)[0].float().view(torch.int32), ref_b):
            moved_b.append(M)
    out["invariance_control_mlp_up_N4096_K1024"] = {
        "row0_bits_differ_from_M2048_at_M": {"gemm_mfma_invariant": moved_m, "hipblaslt": moved_b}}
    del A, W
    # fused epilogue (bias, activation, residual, bf16 output) against the same steps as separate kernels
    F = torch.nn.functional
    N = K = 4096
    WTs = [randn_bf16((N, K), 0.02) for _ in range(16)]
    x8 = randn_bf16((8, K), 1.0)
    bias = torch.randn(N, device="cuda")
    res = torch.randn(8, N, device="cuda")
    for M in (1, 8):
        x, r = x8[:M], res[:M]
        fused = graph_time(lambda i: g.gemv_tree_ep(x, WTs[i % 16], bias=bias, act="silu", residual=r, out="bf16"), 64)
        split = graph_time(lambda i: (F.silu(g.gemv_tree(x, WTs[i % 16]) + bias) + r).to(torch.bfloat16), 64)
        blas = graph_time(lambda i: (F.silu(torch.mm(x, WTs[i % 16].t(), out_dtype=torch.float32) + bias) + r)
                          .to(torch.bfloat16), 64)
        out[f"epilogue_decode_M{M}_silu_bias_residual_bf16"] = {
            "fused_us": round(1e3 * fused, 2), "tree_then_torch_epilogue_us": round(1e3 * split, 2),
            "hipblaslt_then_torch_epilogue_us": round(1e3 * blas, 2)}
    del WTs
    A = randn_bf16((4096, 4096), 1.0)
    W = randn_bf16((4096, 4096), 0.02)
    b2 = torch.randn(4096, device="cuda")
    r2 = torch.randn(4096, 4096, device="cuda")
    gelu = lambda y: F.gelu(y, approximate="tanh")
    fused = graph_time(lambda i: g.gemm_mfma_invariant_ep(A, W, bias=b2, act="gelu_tanh", residual=r2, out="bf16"), 8)
    split = graph_time(lambda i: (gelu(g.gemm_mfma_invariant(A, W) + b2) + r2).to(torch.bfloat16), 8)
    plain = graph_time(lambda i: g.gemm_mfma_invariant(A, W), 8)
    blas = graph_time(lambda i: (gelu(mm_blaslt(A, W) + b2) + r2).to(torch.bfloat16), 8)
    out["epilogue_prefill_4096cube_gelu_bias_residual_bf16"] = {
        "fused_us": round(1e3 * fused, 1), "mfma_then_torch_epilogue_us": round(1e3 * split, 1),
        "mfma_alone_us": round(1e3 * plain, 1), "hipblaslt_then_torch_epilogue_us": round(1e3 * blas, 1)}
    del A, W, r2
    out["certificate_decode_loop_7b_layer"] = cert_loop(g)
    # decode GEMVs at the other projection shapes of a 7B layer (weight as W^T [N, K], 8 rotated copies so
    # that each launch streams its weight from HBM): tree order, the matrix-core GEMV, hipBLASLt
    for N, K in ((11008, 4096), (4096, 11008)):
        WTs = [randn_bf16((N, K), 0.02) for _ in range(8)]
        for M in (1, 8):
            x = randn_bf16((M, K), 1.0)
            rec = {}
            for name, fn in (("tree", lambda i: g.gemv_tree(x, WTs[i % 8])),
                             ("mfma", lambda i: g.gemv_mfma_invariant(x, WTs[i % 8])),
                             ("hipblaslt", lambda i: mm_blaslt(x, WTs[i % 8].t()))):
                t = graph_time(fn, 32)
                rec[f"{name}_us"] = round(1e3 * t, 2)
                rec[f"{name}_GBps"] = round(gemv_bytes(M, K, N) / t / 1e6, 1)
            out[f"decode_gemv_M{M}_N{N}_K{K}"] = rec
        del WTs
    # attention value product, 32 heads, head_dim 128 (L = 5000: P is 3.2 GB, 204.8 GFLOP)
    import numpy as np
    import oracle
    for L in (256, 1024, 5000):
        P = torch.softmax(torch.randn((32, L, L), device="cuda"), dim=-1)
        V = randn_bf16((32, L, 128), 1.0)
        O = torch.empty((32, L, 128), device="cuda")
        t = time_region(lambda: g.gemm_ordered_grouped([(P, V, O)]), max(2, reps // 4), 1)
        flop = 2.0 * 32 * L * L * 128
        # the timed launch's output: rows 0, L/2 and L-1 of the last two heads (head 31 starts past 2^31
        # bytes of P at L = 5000) against the oracle, bit for bit
        torch.cuda.synchronize()
        rows = sorted({0, L // 2, L - 1})
        same = all(np.array_equal(
            O[h, rows].cpu().numpy().view(np.uint32),
            oracle.gemm_ordered(np.ascontiguousarray(P[h, rows].cpu().numpy()),
                                V[h].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)).view(np.uint32))
            for h in (30, 31))
        out[f"pv_L{L}_h32"] = {"ordered_tflops": round(flop / t / 1e9, 2), "ms": round(t, 4),
                               "ordered_frac_contract_peak": round(flop / t / 1e9 / VALU_CONTRACT_PEAK_TFS, 4),
                               "ordered_frac_nominal_peak": round(flop / t / 1e9 / VALU_NOMINAL_PEAK_TFS, 4),
                               "parity_heads_30_31_rows_0_mid_last": "bit-exact" if same else "MISMATCH"}
        del P, V, O
    return out


def cert_loop(g, tokens=48):
    """Decode loop over the seven projections of a 7B layer (q, k, v, o 4096x4096; gate, up 4096->11008;
    down 11008->4096), one row per token through gemv_tree, without and with the certificate engine
    (every output row copied asynchronously and checked on host threads against t sign vectors)."""
    import numpy as np
    import torch
    shapes = [(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)]   # (N, K) of W^T
    WTs = [(torch.randn(n, k, device="cuda") * 0.02).to(torch.bfloat16) for n, k in shapes]
    xs = [[torch.randn(1, k, device="cuda").to(torch.bfloat16) for _ in range(4)] for _, k in shapes]
    res = {"matrices": len(shapes), "tokens": tokens, "rows_per_token": len(shapes)}

    # output rows preallocated, as a serving loop holds them: every row must outlive its copy, and
    # growing the allocator's pool inside the timed loop would time hipMalloc
    outs = [[torch.empty((1, n), device="cuda") for n, _ in shapes] for _ in range(tokens)]

    def run(eng, mids):
        keep, stamps = [], []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for tok in range(tokens):
            stamps.append(time.perf_counter())
            rows = []
            for i in range(len(shapes)):
                x = xs[i][tok % 4]
                y = g.gemv_tree(x, WTs[i], y=outs[tok][i])
                rows.append((x[0], y[0]))
            if eng is not None:            # one gather launch per token for all seven rows
                eng.submit_rows(mids, [r[0] for r in rows], [r[1] for r in rows], token=tok)
                keep.append(rows)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        st = eng.drain() if eng is not None else None
        t2 = time.perf_counter()
        # host time of each token's launches and submit (the device runs behind; the mean includes
        # the final synchronisation)
        per = np.diff(np.array(stamps + [t1]))
        return (t1 - t0) / tokens, t2 - t1, st, float(np.median(per)), float(per.max())

    run(None, None)
    base, _, _, base_med, _ = run(None, None)
    res["no_certificate_us_per_token"] = round(1e6 * base, 1)
    res["no_certificate_median_us_per_token"] = round(1e6 * base_med, 1)
    Wh = [w.view(torch.int16).cpu().numpy().view(np.uint16) for w in WTs]
    for t in (1, 4):
        eng = g.CertEngine(11008, 11008, slots=64, workers=4)
        rng = np.random.default_rng(t)
        mids = [eng.add_matrix(w, rng.choice(np.int8([-1, 1]), size=(t, w.shape[0])), transposed=True) for w in Wh]
        per_tok, drain, st, med, worst = run(eng, mids)
        res[f"t{t}"] = {"us_per_token": round(1e6 * per_tok, 1), "median_us_per_token": round(1e6 * med, 1),
                        "slowest_token_us": round(1e6 * worst, 1), "drain_after_gpu_ms": round(1e3 * drain, 2),
                        "rows_checked": st["checked"], "failed": st["failed"],
                        "max_honest_ratio": round(st["max_honest_ratio"], 5),
                        "host_check_us_per_row": round(1e6 * st["check_seconds"] / max(1, st["checked"]), 1),
                        "copy_wait_us_per_row": round(1e6 * st["wait_seconds"] / max(1, st["checked"]), 1),
                        "submit_wait_us_per_token": round(1e6 * st["submit_wait_seconds"] / tokens, 1),
                        "submit_c_us_per_token": round(1e6 * st["submit_seconds"] / tokens, 1),
                        "escape_probability_of_a_cancelling_fault": 2.0 ** -t}
        eng.close()
    return res


# ---------------------------------------------------------------------------
# HBM traffic of the tree GEMV kernel from rocprofv3 counters.
#
#   rocprofv3 --pmc FETCH_SIZE  ... -- python3 bench.py --counters
#   rocprofv3 --pmc WRITE_SIZE  ... -- python3 bench.py --counters
#   python3 bench.py --traffic-summary <fetch dir> <write dir>
#
# --counters launches a fixed sequence: COPY_REPS plain copies of COPY_BYTES
# (torch's copy kernel: it reads and writes exactly COPY_BYTES), then
# COUNTER_REPS GEMV launches for each M (rotating W). The summary scales each
# GEMV counter value by what the same counter reads for the copy, writes
# profiles/gemv_tree_traffic.json (tagged with the SHA-256 of the kernel
# source) and a markdown summary; the bench reports the traffic only while the
# library's kernel source still has that hash.
# ---------------------------------------------------------------------------
COPY_BYTES = 256 << 20
COPY_REPS = 3
COUNTER_REPS = 4
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "gemv_tree_traffic.json")
GEMV_SOURCE = os.path.join(ROOT, "gemv_gemm_ordered_amd", "csrc", "tree_gemv.hip")
# the counted GEMV kernels: --gemv tree (the headline kernel), mfma (the matrix-core GEMV) or ordered
COUNTED = {
    "tree": {"kernel": "k_gemv_tree_p", "source": "tree_gemv.hip", "json": "gemv_tree_traffic.json",
             "md": "gemv_tree_decode_4096x4096_traffic.md"},
    "mfma": {"kernel": "k_gemv_mfma", "source": "mfma_gemv.hip", "json": "gemv_mfma_traffic.json",
             "md": "gemv_mfma_decode_4096x4096_traffic.md"},
    # gemv_ordered on W [K, N]: k_gemv_ordered at M = 1, k_gemv_ordered_k128 at M = 4 and 8
    "ordered": {"kernel": "k_gemv_ordered, k_gemv_ordered_k128", "source": "ordered_gemv.hip", "json": "gemv_ordered_traffic.json",
                "md": "gemv_ordered_decode_4096x4096_traffic.md"},
}


def source_sha256(name: str) -> str:
    import hashlib
    with open(os.path.join(ROOT, "gemv_gemm_ordered_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def gemv_source_sha256() -> str:
    import hashlib
    with open(GEMV_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def run_counters(which="tree"):
    import numpy as np
    import torch

    import gemv_gemm_ordered_amd as g
    import synth
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    small = src[:(32 << 20) // 4]
    small_dst = dst[:(32 << 20) // 4]
    x, W, _ = synth.decode_gemv(0, 8)
    dx = dev_bf16(x)
    dWs = [dev_bf16(W if which == "ordered" else np.ascontiguousarray(W.T))] + [None] * 3
    for i in range(1, 4):
        dWs[i] = dWs[0].clone()
    ys = {M: torch.empty((M, 4096), device="cuda") for M in (1, 4, 8)}
    torch.cuda.synchronize()
    # calibration kernels, in this order: the runtime's copy blit, a plain
    # elementwise copy (x + 0) of COPY_BYTES, the same of 32 MiB
    for _ in range(COPY_REPS):
        dst.copy_(src)
    torch.cuda.synchronize()
    for _ in range(COPY_REPS):
        torch.add(src, 0.0, out=dst)
    torch.cuda.synchronize()
    for _ in range(COPY_REPS):
        torch.add(small, 0.0, out=small_dst)
    torch.cuda.synchronize()
    i = 0
    gemv = {"tree": g.gemv_tree, "mfma": g.gemv_mfma_invariant, "ordered": g.gemv_ordered}[which]
    for M in (1, 4, 8):
        for _ in range(COUNTER_REPS):
            gemv(dx[:M], dWs[i % 4], y=ys[M])
            i += 1
        torch.cuda.synchronize()
    print("counters sequence done", flush=True)


def _counter_values(directory, counter):
    """Per-dispatch values of `counter` (summed over its instances), in dispatch order, with kernel names."""
    import csv
    import glob
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    per = {}
    for row in csv.DictReader(open(files[0])):
        if row["Counter_Name"] != counter:
            continue
        d = int(row["Dispatch_Id"])
        name, val = row["Kernel_Name"], float(row["Counter_Value"])
        prev = per.get(d, (name, 0.0))
        per[d] = (name, prev[1] + val)
    return [per[d] for d in sorted(per)]


def traffic_summary(fetch_dir, write_dir, which="tree"):
    import statistics
    info = COUNTED[which]
    out = {"source_sha256": source_sha256(info["source"]), "copy_bytes": COPY_BYTES, "units": "bytes per launch",
           "kernel": info["kernel"]}
    for counter, directory in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        seq = _counter_values(directory, counter)
        # the last 3 * COPY_REPS dispatches before the GEMVs are the calibration copies:
        # runtime blit (COPY_BYTES), elementwise copy (COPY_BYTES), elementwise copy (32 MiB)
        others = [v for n, v in seq if "gemv" not in n]
        gemvs = [v for n, v in seq if "gemv" in n]
        if len(others) < 3 * COPY_REPS or len(gemvs) != 3 * COUNTER_REPS:
            raise SystemExit(f"{counter}: unexpected dispatch sequence ({len(others)} others, {len(gemvs)} GEMVs)")
        blit, plain, small = (others[len(others) - 3 * COPY_REPS + i * COPY_REPS:][:COPY_REPS] for i in range(3))
        kib = statistics.median(plain)
        factor = COPY_BYTES / (kib * 1024.0)   # bytes per counted KiB, from the plain elementwise copy
        out[counter] = {"copy_counter_kib": kib, "bytes_per_counted_kib": factor,
                        "check_blit_counter_kib": statistics.median(blit),
                        "check_32MiB_copy_counter_kib": statistics.median(small)}
        for j, M in enumerate((1, 4, 8)):
            vals = gemvs[j * COUNTER_REPS:(j + 1) * COUNTER_REPS]
            out.setdefault("per_M", {}).setdefault(str(M), {})[counter] = {
                "counter_kib": statistics.median(vals), "bytes": statistics.median(vals) * 1024.0 * factor}
    for M, rec in out["per_M"].items():
        rec["algorithmic_bytes"] = gemv_bytes(int(M))
        rec["hbm_bytes"] = rec["FETCH_SIZE"]["bytes"] + rec["WRITE_SIZE"]["bytes"]
        rec["hbm_over_algorithmic"] = rec["hbm_bytes"] / rec["algorithmic_bytes"]
    with open(os.path.join(ROOT, "profiles", info["json"]), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    flag = f" --gemv {which}"
    lines = [f"# {info['kernel']} — HBM traffic per launch (decode GEMV, K = N = 4096)", "",
             "Commands (from the repository root $REPO, on one MI355X; $OUT is any directory for the profiler's output):", "",
             f"    cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/traffic_fetch -o run -- python3 $REPO/bench.py --counters{flag}",
             f"    cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/traffic_write -o run -- python3 $REPO/bench.py --counters{flag}",
             f"    python3 bench.py --traffic-summary $OUT/traffic_fetch $OUT/traffic_write{flag}", "",
             f"Calibration: a plain elementwise copy of {COPY_BYTES >> 20} MiB (reads and writes {COPY_BYTES} "
             f"bytes) reads FETCH_SIZE = {out['FETCH_SIZE']['copy_counter_kib']:.0f} KiB and WRITE_SIZE = "
             f"{out['WRITE_SIZE']['copy_counter_kib']:.0f} KiB, so one counted KiB is "
             f"{out['FETCH_SIZE']['bytes_per_counted_kib']:.3f} KiB fetched and "
             f"{out['WRITE_SIZE']['bytes_per_counted_kib']:.3f} KiB written. Checks: the runtime's copy blit of "
             f"the same size reads {out['FETCH_SIZE']['check_blit_counter_kib']:.0f} / "
             f"{out['WRITE_SIZE']['check_blit_counter_kib']:.0f} KiB, an elementwise copy of 32 MiB "
             f"{out['FETCH_SIZE']['check_32MiB_copy_counter_kib']:.0f} / "
             f"{out['WRITE_SIZE']['check_32MiB_copy_counter_kib']:.0f} KiB.", "",
             "| M | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | HBM bytes (scaled) | algorithmic bytes | ratio |",
             "|---|---|---|---|---|---|"]
    for M, rec in sorted(out["per_M"].items(), key=lambda kv: int(kv[0])):
        lines.append(f"| {M} | {rec['FETCH_SIZE']['counter_kib']:.0f} | {rec['WRITE_SIZE']['counter_kib']:.0f} | "
                     f"{rec['hbm_bytes']:.0f} | {rec['algorithmic_bytes']} | {rec['hbm_over_algorithmic']:.3f} |")
    lines += ["", f"Kernel source ({info['source']}) SHA-256: `{out['source_sha256']}`"
                  + (" (the bench reports `traffic` only for this source)." if which == "tree" else ".")]
    with open(os.path.join(ROOT, "profiles", info["md"]), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic_per_launch(ms):
    """Mean counted HBM bytes per launch over the step's M values, or None if absent or stale."""
    try:
        with open(TRAFFIC_JSON) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != gemv_source_sha256():
        return None
    try:
        return sum(t["per_M"][str(M)]["hbm_bytes"] for M in ms) / len(ms)
    except KeyError:
        return None



# Utilisation counters of the three kinds of kernel (the counter evidence for their design choices):
# the MFMA GEMM at 4096^3, the ordered GEMM at the MLP up-projection (M = 2048), the tree GEMV at M = 8.
# `--counters-kernels` runs KERNEL_REPS launches of each; two rocprofv3 passes collect the counters:
#   rocprofv3 --pmc MfmaUtil SQ_INSTS_MFMA SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_LDS_BANK_CONFLICT ...
#   rocprofv3 --pmc VALUBusy SQ_INSTS_VALU_MUL_F32 SQ_INSTS_VALU_ADD_F32 SQ_INSTS_VALU_FMA_F32 ...
# and `--kernel-counter-summary DIR1 DIR2` writes profiles/utilisation_mfma_4096cube_ordered_mlp_m2048_tree_decode_m8.md.
KERNEL_REPS = 4
KERNEL_PASSES = (
    ("MfmaUtil", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_LDS_BANK_CONFLICT"),
    ("VALUBusy", "SQ_INSTS_VALU_MUL_F32", "SQ_INSTS_VALU_ADD_F32", "SQ_INSTS_VALU_FMA_F32"),
)
KERNEL_WORK = {   # name fragment -> (label, algorithmic flop per launch)
    "k_gemm_mfma_invariant": ("MFMA GEMM 4096x4096x4096", 2.0 * 4096 ** 3),
    "k_gemm_ordered": ("ordered GEMM, MLP up-projection M=2048 N=4096 K=1024", 2.0 * 2048 * 4096 * 1024),
    "k_gemv_tree_p": ("tree GEMV, decode M=8 N=K=4096", 2.0 * 8 * 4096 * 4096),
}


def run_kernel_counters():
    import torch
    import gemv_gemm_ordered_amd as g
    torch.manual_seed(0)
    A = (torch.randn(4096, 4096, device="cuda")).to(torch.bfloat16)
    W = (torch.randn(4096, 4096, device="cuda") * 0.02).to(torch.bfloat16)
    C = torch.empty(4096, 4096, device="cuda")
    for _ in range(KERNEL_REPS):
        g.gemm_mfma_invariant(A, W, C=C)
    A2 = A[:2048, :1024].contiguous()
    W2 = W[:1024].contiguous()
    C2 = torch.empty(2048, 4096, device="cuda")
    for _ in range(KERNEL_REPS):
        g.gemm_ordered(A2, W2, C=C2)
    x = A[:8].contiguous()
    y = torch.empty(8, 4096, device="cuda")
    for _ in range(KERNEL_REPS):
        g.gemv_tree(x, W, y=y)
    torch.cuda.synchronize()
    print("kernel counters sequence done", flush=True)


def kernel_counter_summary(dir1, dir2):
    import csv
    import glob
    import statistics
    rows = {}
    for d in (dir1, dir2):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        for r in csv.DictReader(open(files[0])):
            for frag in KERNEL_WORK:
                if frag in r["Kernel_Name"]:
                    rec = rows.setdefault(frag, {})
                    rec.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                    dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
                    rec.setdefault("_dur", []).append(dur)
    lines = ["# Utilisation counters of the MFMA GEMM, the ordered GEMM and the tree GEMV", "",
             "Commands (from the repository root $REPO, on one MI355X; $OUT is any directory for the profiler's output):", ""]
    for i, p in enumerate(KERNEL_PASSES, 1):
        lines.append(f"    cd /tmp && rocprofv3 --pmc {' '.join(p)} --output-format csv -d $OUT/kcount{i} -o run "
                     "-- python3 $REPO/bench.py --counters-kernels")
    lines += ["    python3 bench.py --kernel-counter-summary $OUT/kcount1 $OUT/kcount2", "",
              f"Medians over {KERNEL_REPS} launches of each kernel. `MfmaUtil` and `VALUBusy` are rocprofv3's "
              "derived metrics (matrix-pipe busy cycles over all SIMDs, and VALU-active cycles per CU, as a "
              "percentage of the GPU-active cycles). Binary32 VALU rate: (mul + add + fma wave instructions) x 64 "
              "lanes over the profiled launch duration, against the 78.6 T op/s of unfused binary32 on 256 CUs "
              "(4 SIMDs x 32 lanes per clock at 2.4 GHz). Durations come from the profiled launches, which run "
              "slower than unprofiled ones.", "",
              "| kernel | MfmaUtil % | VALUBusy % | MFMA instructions | binary32 VALU ops (mul / add / fma, x64 lanes) | "
              "VALU op rate | LDS bank-conflict cycles | profiled duration |",
              "|---|---|---|---|---|---|---|---|"]
    for frag, (label, flop) in KERNEL_WORK.items():
        rec = rows.get(frag)
        if not rec:
            continue
        med = lambda k: statistics.median(rec[k]) if k in rec else float("nan")
        mul, add, fma = med("SQ_INSTS_VALU_MUL_F32"), med("SQ_INSTS_VALU_ADD_F32"), med("SQ_INSTS_VALU_FMA_F32")
        dur = statistics.median(rec["_dur"])
        rate = (mul + add + fma) * 64 / dur / 1e12
        lines.append(f"| {label} (`{frag}`) | {med('MfmaUtil'):.1f} | {med('VALUBusy'):.1f} | {med('SQ_INSTS_MFMA'):.0f} | "
                     f"{mul * 64:.3g} / {add * 64:.3g} / {fma * 64:.3g} | {rate:.1f} T op/s "
                     f"({100 * rate / VALU_CONTRACT_PEAK_TFS:.0f}% of 78.6) | {med('SQ_LDS_BANK_CONFLICT'):.0f} | "
                     f"{1e6 * dur:.1f} us |")
    with open(os.path.join(ROOT, "profiles", "utilisation_mfma_4096cube_ordered_mlp_m2048_tree_decode_m8.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-paths", action="store_true", help="skip the other paths' throughput")
    ap.add_argument("--no-graph", action="store_true", help="eager launches instead of one graph replay")
    ap.add_argument("--gemv", choices=sorted(COUNTED), default="tree",
                    help="which decode GEMV --counters launches and --traffic-summary summarises")
    ap.add_argument("--counters", action="store_true",
                    help="run the fixed launch sequence for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE and exit")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 counter directories into profiles/gemv_tree_traffic.json and exit")
    ap.add_argument("--counters-kernels", action="store_true",
                    help="run the launch sequence for the utilisation counter passes and exit")
    ap.add_argument("--kernel-counter-summary", nargs=2, metavar=("DIR1", "DIR2"),
                    help="turn the two utilisation counter passes into profiles/utilisation_mfma_4096cube_ordered_mlp_m2048_tree_decode_m8.md and exit")
    args = ap.parse_args()
    if args.kernel_counter_summary:
        kernel_counter_summary(*args.kernel_counter_summary)
        return
    if args.counters_kernels:
        run_kernel_counters()
        return
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary, which=args.gemv)
        return
    if args.counters:
        run_counters(args.gemv)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this library's path has no cross-GPU step, and this "
              "benchmark reports one GPU's throughput (--gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gemv_gemm_ordered_amd as g
    import oracle
    import synth

    K = N = 4096
    ms = (1, 4, 8)
    log("generating decode workload")
    x, W, r = synth.decode_gemv(0, 8)
    WT = np.ascontiguousarray(W.T)
    dx = dev_bf16(x)
    copies = 16
    dWT0 = dev_bf16(WT)
    dWTs = [dWT0] + [dWT0.clone() for _ in range(copies - 1)]
    ys = {M: torch.empty((M, N), device="cuda") for M in ms}
    step_bytes = sum(gemv_bytes(M) for M in ms)
    counter = [0]

    def step():
        for M in ms:
            g.gemv_tree(dx[:M], dWTs[counter[0] % copies], y=ys[M])
            counter[0] += 1

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    graph = None
    if args.no_graph:
        run = None
    else:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.steps):
                step()
        run = graph.replay
        run()                       # one untimed replay: uploads the graph
        torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    if run is not None:
        run()
    else:
        for _ in range(args.steps):
            step()
    e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = s.elapsed_time(e)
    ms_per_step = ms_total / args.steps
    value = step_bytes * args.steps / (ms_total / 1e3) / 1e9
    avg_launch_us = 1e3 * ms_total / (args.steps * len(ms))

    # parity spot check of the timed kernel's last outputs against the oracle
    ref = oracle.gemv_tree(x[:8][[0, 7]], WT, threads=4).view(np.uint32)
    got = ys[8].cpu().numpy().view(np.uint32)[[0, 7]]
    parity = "bit-exact (rows 0 and 7 of M=8 vs CPU oracle)" if np.array_equal(got, ref) else "MISMATCH"
    del graph

    # per-M time (64 launches per M, rotating weights, one graph replay each): the tree GEMV, the
    # ordered GEMV on W [K, N] (the one-lane chain contract) and hipBLASLt (not batch invariant)
    dW0 = dev_bf16(W)
    dWs = [dW0] + [dW0.clone() for _ in range(copies - 1)]
    per_m = {}
    for M in ms:
        rec = {}
        for name, fn in (("tree", lambda i: g.gemv_tree(dx[:M], dWTs[i % copies], y=ys[M])),
                         ("mfma", lambda i: g.gemv_mfma_invariant(dx[:M], dWTs[i % copies], y=ys[M])),
                         ("ordered", lambda i: g.gemv_ordered(dx[:M], dWs[i % copies], y=ys[M])),
                         ("ordered_wt", lambda i: g.gemv_ordered_wt(dx[:M], dWTs[i % copies], y=ys[M])),
                         ("hipblaslt", lambda i: torch.mm(dx[:M], dWTs[i % copies].t(), out_dtype=torch.float32))):
            try:
                t = graph_time(fn, 64)
            except RuntimeError as err:      # a library that cannot be captured is timed eagerly
                log(f"{name} M={M}: graph capture failed ({err}); eager timing")
                i = [0]

                def one():
                    fn(i[0])
                    i[0] += 1
                t = time_region(one, 64)
            rec[name] = {"us": round(1e3 * t, 2), "GBps": round(gemv_bytes(M) / t / 1e6, 1),
                         "frac_hbm": round(gemv_bytes(M) / t / 1e6 / HBM_PEAK_GBS, 4)}
        per_m[str(M)] = rec
    del dWs

    cert = certificate(g, x, W, r, ys, ms)
    extra = {} if args.no_paths else paths(g, 10)
    log("cpu baseline")
    cpu = cpu_baseline(x, WT, ms, args.cpu_seconds)
    log("cpu oracle on the other workloads")
    cpu["configs"] = cpu_oracle_configs(max(0.2, args.cpu_seconds / 10))

    achieved = (step_bytes / len(ms)) / (avg_launch_us * 1e-6) / 1e9
    line = {
        "metric": "batch-invariant GEMM TFLOP/s & GEMV GB/s vs M, bit-exact; % of roofline",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded splitmix64/Box-Muller; x ~ N(0,1), W ~ N(0,0.02), bf16)",
        "config": {"workload": "decode GEMV, gemv_tree: x[M,4096] bf16 x W^T[4096,4096] bf16 -> y f32, "
                               "M in {1,4,8} per step, 16 rotated weight copies",
                   "K": K, "N": N, "M_per_step": list(ms), "w_copies": copies,
                   "graph": run is not None, "parity": parity},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_per_launch(ms),
                     "kernel": "k_gemv_tree_p", "avg_launch_us": round(avg_launch_us, 3),
                     "bytes_per_launch": step_bytes / len(ms)},
        "cpu_baseline": cpu,
        "per_M": per_m,
        "certificate": cert,
        "paths": extra,
        "wall_s_timed": round(wall, 4),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
