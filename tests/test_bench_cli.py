"""bench.py's command-line contract and its host-side helpers (no GPU)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def run_bench(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, timeout=timeout, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert b"one GPU" in r.stderr
    assert r.stdout == b""


def test_no_gpu_exits_with_a_message():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = run_bench("--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert b"GPU" in r.stderr
    assert r.stdout == b""


def test_per_expert_roofline_closed_forms():
    import bench
    D, F = 6144, 2048
    B = 18_915_328                       # one int4 expert's weights and scales
    hbm = B / (bench.HBM_PEAK_GBS * 1e9)
    flop = lambda r: 2.0 * r * 3 * D * F / (bench.BF16_PEAK_TFLOPS * 1e12)
    # unused experts cost nothing; a one-row expert is bound by its bytes
    assert bench.per_expert_roofline_s([0, 0], B, D, F) == 0.0
    assert bench.per_expert_roofline_s([1], B, D, F) == pytest.approx(hbm)
    # a large expert is bound by its flops; experts add
    assert bench.per_expert_roofline_s([4096], B, D, F) == pytest.approx(flop(4096))
    assert bench.per_expert_roofline_s([1, 4096, 0, 1], B, D, F) == pytest.approx(2 * hbm + flop(4096))
    # the crossover row count sits where bytes and flops take equal time
    r_star = B / (bench.HBM_PEAK_GBS * 1e9) * (bench.BF16_PEAK_TFLOPS * 1e12) / (2.0 * 3 * D * F)
    assert 70 < r_star < 85
    lo, hi = int(r_star), int(r_star) + 1
    assert bench.per_expert_roofline_s([lo], B, D, F) == pytest.approx(hbm)
    assert bench.per_expert_roofline_s([hi], B, D, F) == pytest.approx(flop(hi))


def test_host_info_reports_cpus_and_model():
    import bench
    n, model = bench.host_info()
    assert n >= 1
    assert isinstance(model, str) and model


def test_oracle_thread_count_changes_no_value():
    """The oracle splits work over rows or tokens, one thread per result, so
    one thread and all threads give the same bits; set_threads restores."""
    import numpy as np
    from oracle import oracle
    from weight_streaming_gemv_qgemv_amd import synth
    g = synth.rng(9100)
    O, I, S = 37, 512, 3
    W = synth.weight_bytes(g, 2, O, I)
    sc = synth.scales(g, O)
    x = synth.activations(g, S, I)
    Wr, bias = synth.router_weights(g, 16, I)
    y_all, _ = oracle.qgemv(2, W, sc, x)
    r_all = oracle.router(Wr, bias, x, 4, 1, 2.5)
    prev = oracle.set_threads(1)
    try:
        assert oracle.num_threads() == 1
        y_one, _ = oracle.qgemv(2, W, sc, x)
        r_one = oracle.router(Wr, bias, x, 4, 1, 2.5)
    finally:
        assert oracle.set_threads(prev) == 1
    assert oracle.num_threads() == prev
    assert np.array_equal(y_all, y_one)
    assert np.array_equal(r_all["idx"], r_one["idx"])
    assert np.array_equal(r_all["w"], r_one["w"])
