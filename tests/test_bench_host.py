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


def _csv(path, header, rows):
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=header)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_profile_summary_counts_dispatches_per_call(tmp_path, monkeypatch):
    """A call made of two dispatches (main launch + ragged-tail launch): the renamed
    trace row holds 2 dispatches per timed call, and the copy-calibrated traffic of
    one call is twice the per-dispatch mean."""
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    d = tmp_path / "prof"
    stats_h = ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"]
    _csv(str(d / "trace" / "t_kernel_stats.csv"), stats_h,
         [dict(Name="timed: contiguous X", Calls=10, AverageNs=400000, MinNs=1, MaxNs=2)])
    ctr_h = ["Kernel_Name", "Dispatch_Id", "Counter_Name", "Counter_Value"]
    for sub, name, gemm_vals, copy_val in (("fetch", "FETCH_SIZE", [1000.0, 3000.0], 131072.0),
                                           ("write", "WRITE_SIZE", [500.0, 500.0], 262144.0)):
        rows = [dict(Kernel_Name="__amd_rocclr_copyBuffer", Dispatch_Id=1, Counter_Name=name, Counter_Value=copy_val)]
        rows += [dict(Kernel_Name="void dg::gemm_kernel<256>", Dispatch_Id=2 + i, Counter_Name=name, Counter_Value=v)
                 for i, v in enumerate(gemm_vals)]
        _csv(str(d / sub / "x_counter_collection.csv"), ctr_h, rows)
    line = dict(steps=5, value=1.0, unit="TFLOPS",
                roofline=dict(avg_launch_us=800.0, achieved=1.0, unit="TFLOP/s", frac=0.1))
    (d / "bench_line.json").write_text(json.dumps(line) + "\n")
    out = tmp_path / "s.md"
    bench.profile_summary(str(d), str(out), "contiguous X", "cmd")
    text = out.read_text()
    assert "2 dispatches per call (5 timed calls): 800.0 us per call" in text
    rec = json.loads((tmp_path / "traffic.json").read_text())["cases"]["contiguous X"]
    # factors: 131072 KiB / 256 MiB = 0.5 (fetch), 262144 KiB / 256 MiB = 1.0 (write)
    assert abs(rec["traffic_bytes"] - 2 * (2000 * 1024 / 0.5 + 500 * 1024 / 1.0)) < 1e-6


def test_counter_summary_derives_clock_and_busy(tmp_path):
    """GRBM_GUI_ACTIVE is summed over 8 XCDs: 8 x 1.9e9 x 200 us over a 200 us dispatch is
    1.9 GHz; busy cycles equal to half of 1024 SIMDs x those cycles is 0.5 busy."""
    d = tmp_path / "ctr"
    cyc = 1.9e9 * 200e-6
    busy = 0.5 * cyc * 1024
    flops = busy / 32 * (2 * 16 * 16 * 128)
    h = ["Kernel_Name", "Dispatch_Id", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    rows = [dict(Kernel_Name="gemm_kernel<256, 256", Dispatch_Id=1, Counter_Name="GRBM_GUI_ACTIVE",
                 Counter_Value=8 * cyc, Start_Timestamp=1000, End_Timestamp=201000),
            dict(Kernel_Name="gemm_kernel<256, 256", Dispatch_Id=1, Counter_Name="SQ_VALU_MFMA_BUSY_CYCLES",
                 Counter_Value=busy, Start_Timestamp=1000, End_Timestamp=201000)]
    _csv(str(d / "p1" / "p_counter_collection.csv"), h, rows)
    out = tmp_path / "c.md"
    bench.counter_summary(str(d), str(out), "case", "cmd", "gemm_kernel<256, 256", flops, 190.0)
    text = out.read_text()
    assert "SQ_VALU_MFMA_BUSY_CYCLES per algorithmic MFMA: 32.00" in text
    assert "dispatch duration: 1.90 GHz" in text
    assert "SIMDs): 0.500" in text


def _last_json_line(path):
    with open(path) as f:
        return json.loads(f.read().strip().splitlines()[-1])


def test_committed_bench_lines_keep_the_output_contract():
    """Every committed bench line carries the fields the JSON contract names, with a
    roofline object whose fraction follows from its own numbers; the default line also
    carries the CPU-oracle baseline and a measured traffic figure."""
    import glob

    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "bench_*.json")))
    assert any(p.endswith("bench_baseline.json") for p in paths)
    for p in paths:
        d = _last_json_line(p)
        name = os.path.basename(p)
        for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                    "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
            assert key in d, (name, key)
        assert d["n_gpus"] == 1 and d["higher_is_better"] is True and d["scaling"] == "weak", name
        assert d["vs_baseline"] is None and d["value"] > 0 and d["ms_per_step"] > 0, name
        assert "workload" in d["config"] and "model" not in d["config"], name
        r = d["roofline"]
        assert r["bound"] in ("mfma", "hbm") and r["unit"] == ("TFLOP/s" if r["bound"] == "mfma" else "GB/s"), name
        assert r["peak"] == (5000.0 if r["bound"] == "mfma" else 8000.0), name
        assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9 and 0 < r["frac"] < 1, name
        assert r["traffic"] is None or r["traffic"] > 0, name
        cpu = d["cpu_baseline"]
        if cpu is not None:
            assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0 and cpu["sample"], name
    base = _last_json_line(os.path.join(ROOT, "profiles", "bench_baseline.json"))
    assert base["config"]["workload"] == "baseline" and base["cpu_baseline"] is not None
    assert base["roofline"]["traffic"] is not None
    assert base["steps"] == 5 and base["warmup"] == 2  # the defaults the driver runs
