"""CPU: bench.py's command line and the arithmetic of its figures (no GPU)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_help_lists_the_modes():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--probe", "--probe-rows", "--all", "--no-cpu-baseline"):
        assert flag in r.stdout


def test_kernel_stats_rates():
    # 1 GiB of algorithmic bytes in 200 us per launch: 5368.7 GB/s; an AllReduce's
    # bus bandwidth of S = 128 MiB per rank over the same time, times 2(P-1)/P
    st = bench.kernel_stats([190.0, 200.0, 210.0], 1 << 30, 128 << 20, 2 * 7 / 8)
    assert st["mean_us"] == pytest.approx(200.0)
    assert st["median_us"] == pytest.approx(200.0)
    assert st["hbm_GBps"] == pytest.approx(round((1 << 30) / 200e-6 / 1e9, 1))
    assert st["busbw_GBps"] == pytest.approx(round((128 << 20) / 200e-6 / 1e9 * 1.75, 1))
    assert st["p10_us"] <= st["median_us"] <= st["p90_us"]


def test_kernel_source_hash_is_stable():
    assert bench.kernel_source_hash() == bench.kernel_source_hash()
    assert len(bench.kernel_source_hash()) == 16


def test_host_cpu_model_is_a_string():
    assert isinstance(bench.host_cpu_model(), str)


def test_alpha_beta_fit_by_regime():
    """Points made from alpha = 3 us, a cache-resident rate of 9 TB/s and an
    HBM rate of 6 TB/s: the fit recovers each, and the HBM figure never
    exceeds the best measured HBM point."""
    p, alpha = 16, 3e-6
    sizes = [4 ** k for k in range(6, 16)]
    us = []
    for s in sizes:
        b = 9e12 if 2 * p * s <= bench.MALL_BYTES else 6e12
        t = alpha + 2 * p * s / b
        us.append(t * 1e6)
    fit = bench.alpha_beta_fit(sizes, us, p)
    assert fit["alpha_us"] == pytest.approx(sum(us[:3]) / 3, abs=1e-3)
    assert fit["hbm"]["points"] == 3  # 64 MiB, 256 MiB and 1 GiB per rank
    assert fit["hbm"]["B_GBps"] <= fit["hbm"]["best_point_GBps"] * 1.01
    assert fit["hbm"]["B_GBps"] == pytest.approx(6000, rel=0.01)
    assert fit["cache"]["points"] == 2  # 1 MiB and 4 MiB per rank (256 KiB takes under 2 alpha)
    assert fit["cache"]["B_GBps"] == pytest.approx(9000, rel=0.05)
    # measured-looking points: the HBM figure stays within the measured rates
    us2 = [3.5, 3.6, 4.0, 5.2, 7.0, 14.0, 95.0, 356.0, 1371.0, 5718.0]
    fit2 = bench.alpha_beta_fit(sizes, us2, p)
    assert fit2["hbm"]["B_GBps"] <= fit2["hbm"]["best_point_GBps"]
