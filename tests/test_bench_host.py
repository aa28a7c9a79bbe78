"""CPU tests of the benchmark's host logic: algorithmic work counts and the
CPU-oracle baseline on tiny inputs (no GPU)."""

import json
import subprocess
import sys
import os

import numpy as np

import bench
from workloads import gen_contiguous, gen_dense, gen_k_grouped, gen_masked, gen_mqa, gen_quant_input

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_work_counts():
    x = gen_dense(64, 256, 512, seed=1)
    f, b = bench.algorithmic_work(x)
    assert f == 2.0 * 64 * 256 * 512
    assert b == 64 * 512 + 256 * 512 + 4 * 64 * 4 + 4 * 2 * 4 + 64 * 256 * 2
    xu = gen_dense(64, 256, 1024, seed=1, scale_fmt="ue8m0")
    assert bench.algorithmic_work(xu)[1] == 64 * 1024 + 256 * 1024 + 4 * 64 * 2 + 4 * 2 * 2 + 64 * 256 * 2
    c = gen_contiguous(3, 256, 256, seed=2, m_sizes=[100, 0, 130])
    f, _ = bench.algorithmic_work(c)
    assert f == 2.0 * 230 * 256 * 256  # padding rows and empty groups do no work
    m = gen_masked(3, 64, 128, 256, seed=3, masked_m=[10, 0, 99])
    assert bench.algorithmic_work(m)[0] == 2.0 * (10 + 64) * 128 * 256  # masked_m clamped to M_max
    k = gen_k_grouped(2, 128, 256, seed=4, ks=[256, 128])
    assert bench.algorithmic_work(k)[0] == 2.0 * 128 * 256 * 384
    q = gen_mqa(8, 40, 16, 128, seed=5, ranges="causal")
    pairs = sum(40 - 8 + i + 1 for i in range(8))
    assert bench.algorithmic_work(q)[0] == 2.0 * 16 * 128 * pairs
    t = dict(kind="quant_token", m=10, k=256, dtype="bf16", x=None)
    assert bench.algorithmic_work(t) == (0.0, 10 * 256 * 3 + 10 * 2 * 4)


def test_cpu_baseline_reports_oracle_rates():
    r = bench.cpu_baseline([gen_dense(32, 128, 256, seed=6)])
    assert r["kind"] == "oracle" and r["unit"] == "TFLOPS" and r["value"] > 0 and r["cores"] >= 1
    r = bench.cpu_baseline([dict(kind="quant_block", m=130, k=256, dtype="fp32",
                                 x=gen_quant_input(130, 256, seed=7, dtype="fp32"))])
    assert r["unit"] == "GB/s" and r["value"] > 0


def test_bench_refuses_more_than_one_gpu():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT)
    assert p.returncode != 0 and "one GPU" in p.stderr
