"""Host-side logic of bench.py (CPU only): the algorithmic bytes and flops of
a call, its roofline time, the roofline object of the dominant kernel, and
the refusal of more than one GPU."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
bench = pytest.importorskip("bench")


def test_tq1_row_bytes():
    # ceil(K / 5) rounded up to 16: 1639 -> 1648 at K = 8192
    assert bench.tq1_ldq(8192) == 1648
    assert bench.tq1_ldq(256) == 64
    assert bench.tq1_ldq(1280) == 256


def test_algorithmic_bytes_and_roofline_times():
    K, N = 8192, 8192
    # TQ2 at M = 1: N K / 4 weight bytes, 2 N K / 256 scale bytes, X and Y
    assert bench.alg_bytes("tq2", 1, N, K) == N * K // 4 + 2 * N * 32 + 2 * K + 2 * N
    assert bench.alg_bytes("tq2", 1, N, K) == 17_334_272
    # TQ1: N ldq weight bytes, same scales
    assert bench.alg_bytes("tq1", 1, N, K) == N * 1648 + 2 * N * 32 + 2 * K + 2 * N
    # the backward moves dY and dX of the same sizes as X and Y
    assert bench.alg_bytes("bwd", 4096, N, K) == bench.alg_bytes("tq2", 4096, N, K)
    assert bench.alg_flops(128, 28672, 8192) == 2 * 128 * 28672 * 8192
    # M = 1 is HBM-bound (17.33 MB at 8 TB/s = 2.167 us), M = 128 at N = 28672
    # MFMA-bound (60.1 GFLOP at 2.5 PFLOP/s = 24.05 us): the worked figures
    assert abs(bench.t_roof("tq2", 1, N, K) - 17_334_272 / 8e12) < 1e-15
    t = bench.t_roof("tq2", 128, 28672, 8192)
    assert abs(t - 2 * 128 * 28672 * 8192 / 2.5e15) < 1e-15
    # the ridge: bytes / 8e12 = flops / 2.5e15 near M = 40 at 0.2578 B/weight
    # (a little higher, ~43, once the bytes of X and Y are counted)
    below = bench.t_roof("tq2", 40, N, K) == bench.alg_bytes("tq2", 40, N, K) / 8e12
    above = bench.t_roof("tq2", 48, N, K) == bench.alg_flops(48, N, K) / 2.5e15
    assert below and above


def test_workload_is_the_sweep():
    calls = bench.workload_calls()
    assert len(calls) == 2 * 8 + 2 * 4
    assert {c[1] for c in calls if c[0] == "tq2"} == {1, 2, 4, 8, 16, 32, 64, 128}
    assert {c[1] for c in calls if c[0] == "tq1"} == {1, 4, 16, 64}
    assert {(c[3], c[2]) for c in calls} == {(8192, 8192), (8192, 28672)}


def test_roofline_of_picks_the_dominant_kernel():
    mk = lambda fmt, M, N, kernel, us: {"fmt": fmt, "M": M, "N": N, "K": 8192,
                                        "kernel": kernel, "us": us}
    calls = [mk("tq2", 1, 8192, "a", 10.0), mk("tq2", 2, 8192, "a", 10.0),
             mk("tq2", 128, 28672, "b", 15.0)]
    r = bench.roofline_of(calls)
    assert r["kernel"] == "a" and r["bound"] == "hbm" and r["launches_per_step"] == 2
    nbytes = bench.alg_bytes("tq2", 1, 8192, 8192) + bench.alg_bytes("tq2", 2, 8192, 8192)
    assert abs(r["achieved"] - round(nbytes / 20e-6 / 1e9, 2)) < 0.01
    assert r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    r2 = bench.roofline_of([mk("tq2", 128, 28672, "b", 30.0)])
    assert r2["bound"] == "mfma" and r2["unit"] == "TFLOP/s" and r2["peak"] == 2500.0


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert out.returncode == 2
    assert "one GPU" in out.stderr
    assert out.stdout == ""
