#!/usr/bin/env python3
"""Benchmark of the fine-grained-scaled FP8 GEMM library on one MI355X.

One step = one pass of the selected workload through the library's C ABI,
with inputs already resident in HBM.  The default workload ("baseline") is
the five benchmark configurations, 20 calls: (0) dense M=128 N=256 K=512;
(1) the 15-shape dense sweep, M in {64, 128, 4096} x (N, K) in {(2112,7168),
(24576,1536), (7168,16384), (4096,7168), (7168,2048)}; (2) the contiguous MoE
GEMM, 8 groups of U[1,8192] tokens, N=4096 K=7168; (3) masked decode, 16
groups of U[0,256] rows, (N,K) in {(4096,7168), (7168,2048)}; (4) dense
M=N=8192 K=16384 with FP32 C and D.  BF16 out except (4).  Prints ONE JSON line:

  value        whole-job FP8 TFLOPS = algorithmic flops of the step / wall time
  roofline     the dominant launch (largest per-launch time) against the MI355X
               dense-FP8 MFMA peak (or HBM bandwidth when that binds), timed
               with HIP events on the stream the library launches on
  cpu_baseline the FP64 CPU oracle on a bounded sample of the same workload
  detail       per-shape cold/warm times, TFLOPS and roofline fractions, and per
               configuration the cold TFLOPS (sum of flops / sum of cold times)

Algorithmic work counts only what the method must do: flops 2*N*K per valid
row; bytes = A (valid rows) + B (groups with valid rows) + scales + D (valid
rows) (+ C).  Padding rows and masked rows are never counted.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0  # MI355X dense FP8 MFMA, published (no sparsity)
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E, published
CSRC = os.path.join(ROOT, "moe_grouped_gemm_tiles_amd", "csrc")
# Sources whose change invalidates a traffic record, per kernel family.
KERNEL_SOURCES = {
    "gemm": ["dg_kernels.hpp", "dg_api.hip", "dg_common.hpp"],
    "quant": ["dg_quant.hip", "dg_common.hpp"],
    "mqa": ["dg_mqa.hip", "dg_common.hpp"],
}


def kernel_family(case_label: str) -> str:
    if case_label.startswith("mqa"):
        return "mqa"
    if "cast" in case_label:
        return "quant"
    return "gemm"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_CAL_MB = 256  # plain device-to-device copy used to calibrate FETCH_SIZE / WRITE_SIZE
TIMED_MARK = "timed: "  # roctx range name prefix of the timed launches of the dominant case


def strip_comments(src: str) -> str:
    """C/C++ source without comments and with runs of whitespace collapsed (string
    and character literals kept), so that editing a comment does not change the hash."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(family: str) -> str:
    """Hash of the sources of a kernel family, comments and whitespace excluded."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family]:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(strip_comments(fh.read()).encode())
    return h.hexdigest()[:16]


def lookup_traffic(case_label: str):
    """HBM bytes per launch measured with rocprofv3 counters for this kernel source, or None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get("cases", {}).get(case_label)
    if ent is None or ent.get("source_hash") != kernel_source_hash(kernel_family(case_label)):
        return None  # no record, or the kernel changed since the counters were taken
    return ent.get("traffic_bytes")


def counter_summary(prof_dir: str, out_md: str, case_label: str, command: str, kernel: str, flops: float,
                    launch_us: float, cus: int = 256, xcds: int = 8):
    """Summarise rocprofv3 --pmc runs (every */*counter_collection.csv under prof_dir) for one kernel:
    the mean of each counter per dispatch, and, where the counters are there, the ratios they give."""
    import csv
    import glob

    per, dur, ratio = {}, {}, []
    for f in glob.glob(os.path.join(prof_dir, "**", "*counter_collection.csv"), recursive=True):
        rows = [r for r in csv.DictReader(open(f)) if kernel in r["Kernel_Name"]]
        for r in rows:
            per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            dur[(f, r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                ratio.append(float(r["Counter_Value"]) / dur[(f, r["Dispatch_Id"])])
    mean = {k: sum(v) / len(v) for k, v in per.items()}
    mean_dur = sum(dur.values()) / len(dur) if dur else 0.0
    lines = [f"# rocprofv3 counters: {case_label}", "", "Command (run from the repository root):", "", "```",
             command, "```", "", f"Kernel: `{kernel}`; mean per dispatch over the dispatches of the run.", "",
             "| counter | dispatches | mean per dispatch |", "|---|---:|---:|"]
    for k in sorted(mean):
        lines.append(f"| {k} | {len(per[k])} | {mean[k]:.4g} |")
    lines += ["", "## Derived", ""]
    mfma = flops / (2 * 16 * 16 * 128)  # v_mfma_f32_16x16x128_f8f6f4 instructions of the algorithmic work
    if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
        lines.append(f"- 16x16x128 FP8 MFMAs of the algorithmic work: {mfma:.4g}; SQ_VALU_MFMA_BUSY_CYCLES per "
                     f"algorithmic MFMA: {mean['SQ_VALU_MFMA_BUSY_CYCLES'] / mfma:.2f} (32 when the kernel "
                     f"multiplies no padding, masked or tile-rounding rows)")
    lines.append(f"- dispatch duration under the counter runs: {mean_dur * 1e6:.1f} us "
                 f"(the same launch unprofiled, from the bench line: {launch_us:.1f} us)")
    if ratio and mean_dur < 100e-6:
        lines.append("- GRBM_GUI_ACTIVE over dispatches this short does not give the clock (the counter window "
                     "is wider than the dispatch timestamps); no clock or busy fraction derived")
        ratio = []
        mean.pop("GRBM_GUI_ACTIVE")
    if ratio:
        lines.append(f"- GRBM_GUI_ACTIVE (summed over the {xcds} XCDs) / {xcds} / dispatch duration: "
                     f"{sum(ratio) / len(ratio) / xcds / 1e9:.2f} GHz (the clock the kernel ran at)")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
            busy = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (mean["GRBM_GUI_ACTIVE"] / xcds * 4 * cus)
            lines.append(f"- SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {xcds} x {4 * cus} SIMDs): {busy:.3f} "
                         f"(the matrix cores were busy that fraction of the kernel's cycles)")
    if "SQ_LDS_BANK_CONFLICT" in mean and "SQ_LDS_IDX_ACTIVE" in mean and mean["SQ_LDS_IDX_ACTIVE"] > 0:
        lines.append(f"- SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE: "
                     f"{mean['SQ_LDS_BANK_CONFLICT'] / mean['SQ_LDS_IDX_ACTIVE']:.4f}")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def profile_summary(prof_dir: str, out_md: str, case_label: str, command: str, kernel: str = "gemm_kernel"):
    """Summarise rocprofv3 output (trace/, fetch/, write/ under prof_dir) into a short text file and
    record the calibrated HBM traffic of the GEMM kernel in profiles/traffic.json."""
    import csv
    import glob

    def rows(sub, pat):
        files = glob.glob(os.path.join(prof_dir, sub, "**", pat), recursive=True)
        return [r for f in files for r in csv.DictReader(open(f))]

    stats = rows("trace", "*kernel_stats.csv")
    counters = {}
    for sub, name in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        per = {}
        for r in rows(sub, "*counter_collection.csv"):
            if r["Counter_Name"] == name:
                per.setdefault(r["Kernel_Name"], []).append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
        counters[name] = per

    def mean_of(per, pred):
        vals = [v for k, vs in per.items() if pred(k) for _, v in vs]
        return sum(vals) / len(vals) if vals else None

    def first_of(per, pred):
        # the calibration copy is the process's first copy dispatch (input uploads come later)
        vals = sorted((d, v) for k, vs in per.items() if pred(k) for d, v in vs)
        return vals[0][1] if vals else None

    is_gemm = lambda k: kernel in k
    is_copy = lambda k: "copy" in k.lower() and kernel not in k
    cal_bytes = COPY_CAL_MB * (1 << 20)
    f_gemm = mean_of(counters["FETCH_SIZE"], is_gemm)
    w_gemm = mean_of(counters["WRITE_SIZE"], is_gemm)
    f_copy = first_of(counters["FETCH_SIZE"], is_copy)
    w_copy = first_of(counters["WRITE_SIZE"], is_copy)
    lines = [f"# rocprofv3 summary: {case_label}", "", "Command (run from the repository root):", "", "```",
             command, "```", "", "## Kernel trace (--kernel-trace --stats)", "",
             "| kernel | calls | avg us | min us | max us |", "|---|---:|---:|---:|---:|"]
    for r in stats:
        lines.append(f"| {r['Name'][:110]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    timed = [r for r in stats if r["Name"].startswith(TIMED_MARK)]
    per_call = 1  # kernel dispatches per library call (a contiguous call with a split tail makes two)
    if timed:
        r = timed[0]
        lines += ["", "## Timed launches of the dominant case", "",
                  f"- rocprofv3 (launches inside the `{r['Name'][:80]}` roctx range, renamed by "
                  f"`--kernel-rename`): {r['Calls']} calls, average {float(r['AverageNs']) / 1e3:.1f} us"]
        try:
            with open(os.path.join(prof_dir, "bench_line.json")) as f:
                line = json.loads([t for t in f.read().splitlines() if t.startswith("{")][-1])
            roof = line["roofline"]
            per_call = max(1, round(int(timed[0]["Calls"]) / int(line["steps"])))
            if per_call > 1:
                lines.append(f"- {per_call} dispatches per call ({line['steps']} timed calls): "
                             f"{per_call * float(timed[0]['AverageNs']) / 1e3:.1f} us per call")
            lines.append(f"- the same run's bench line (HIP events on the launch stream): "
                         f"{roof['avg_launch_us']:.1f} us per launch, {roof['achieved']:.1f} {roof['unit']}, "
                         f"frac {roof['frac']:.3f}; value {line['value']:.1f} {line['unit']}")
        except (OSError, ValueError, KeyError, IndexError):
            lines.append("- bench line of the profiled run: not found")
    traffic = None
    lines += ["", "## HBM traffic (--pmc FETCH_SIZE, then --pmc WRITE_SIZE; KiB per dispatch)", ""]
    if None not in (f_gemm, w_gemm, f_copy, w_copy):
        kf = f_copy * 1024 / cal_bytes
        kw = w_copy * 1024 / cal_bytes
        traffic = (f_gemm * 1024 / kf + w_gemm * 1024 / kw) * per_call
        lines += [f"- copy calibration ({COPY_CAL_MB} MiB device copy): FETCH_SIZE {f_copy:.0f} KiB "
                  f"(factor {kf:.3f}), WRITE_SIZE {w_copy:.0f} KiB (factor {kw:.3f})",
                  f"- `{kernel}`: FETCH_SIZE {f_gemm:.0f} KiB, WRITE_SIZE {w_gemm:.0f} KiB per dispatch",
                  f"- calibrated HBM traffic per launch: {traffic / 1e6:.1f} MB"
                  + (f" ({per_call} dispatches of the mean above)" if per_call > 1 else "")]
        rec = {}
        try:
            rec = json.load(open(TRAFFIC_FILE))
        except (OSError, ValueError):
            pass
        rec.setdefault("cases", {})
        rec.pop("source_hash", None)
        rec["cases"][case_label] = {"traffic_bytes": traffic, "fetch_kib": f_gemm, "write_kib": w_gemm,
                                    "fetch_factor": kf, "write_factor": kw,
                                    "source_hash": kernel_source_hash(kernel_family(case_label))}
        os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(rec, f, indent=1)
    else:
        lines.append("- counters missing")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


class _RangeMarks:
    """roctx ranges around the timed launches of the dominant case, so that a
    ``rocprofv3 --kernel-trace --kernel-rename`` run of this same command reports those
    launches as their own row. Outside a profiler the calls are no-ops; without the
    library the marks are skipped (they only label a trace)."""

    def __init__(self):
        import ctypes
        self._lib = None
        for name in ("librocprofiler-sdk-roctx.so.1", "/opt/rocm/lib/librocprofiler-sdk-roctx.so.1"):
            try:
                lib = ctypes.CDLL(name)
                break
            except OSError:
                continue
        else:
            return
        lib.roctxRangePushA.argtypes = [ctypes.c_char_p]
        lib.roctxRangePushA.restype = ctypes.c_int
        lib.roctxRangePop.argtypes = []
        lib.roctxRangePop.restype = ctypes.c_int
        self._lib = lib

    def push(self, msg: str):
        if self._lib is not None:
            self._lib.roctxRangePushA(msg.encode())

    def pop(self):
        if self._lib is not None:
            self._lib.roctxRangePop()



def _cdiv(a, b):
    return (a + b - 1) // b


def algorithmic_work(x: dict):
    """(flops, bytes) the method must do for one call on inputs ``x``."""
    import numpy as np
    if x["kind"] == "mqa":
        lo = np.clip(x["ks"], 0, x["s_kv"])
        hi = np.clip(x["ke"], 0, x["s_kv"])
        pairs = float(np.maximum(hi - lo, 0).sum())
        s, h, d, s_kv = x["s"], x["h"], x["d"], x["s_kv"]
        # q, kv, scales, weights, ranges in; every logit out (clean_logits fills -inf)
        return 2.0 * h * d * pairs, s * h * d + s_kv * d + 4 * s_kv + 4 * s * h + 8 * s + 4 * s * s_kv
    if x["kind"] in ("quant_token", "quant_block"):
        m, k = x["m"], x["k"]
        es = 2 if x["dtype"] == "bf16" else 4
        scales = m * (k // 128) * 4 if x["kind"] == "quant_token" else _cdiv(m, 128) * (k // 128) * 4
        return 0.0, m * k * es + m * k + scales
    k = x["k"]
    # scale entries per row along K: FP32 per 128-K block, or packed UE8M0 words
    kb = _cdiv(k // 128, 4) if x.get("scale_fmt") == "ue8m0" else k // 128
    out_b = 2 if x.get("out_dtype", "fp32") == "bf16" else 4
    n = x["n"]
    nb = _cdiv(n, 128)
    if x["kind"] == "k_grouped":
        m, g = x["m"], x["num_groups"]
        c_b = g * m * n * 4 if x.get("c") is not None else 0
        return 2.0 * m * n * k, m * k + n * k + 4 * m * kb + 4 * nb * kb + g * m * n * 4 + c_b
    if x["kind"] == "dense":
        m = x["m"]
        c_b = m * n * out_b if x.get("c") is not None else 0
        return 2.0 * m * n * k, m * k + n * k + 4 * m * kb + 4 * nb * kb + m * n * out_b + c_b
    if x["kind"] == "contiguous":
        sizes = np.asarray(x["m_sizes"])
        rows = int(sizes.sum())
        groups = int((sizes > 0).sum())
    else:
        sizes = np.clip(np.asarray(x["masked_m"]), 0, x["m_max"])
        rows = int(sizes.sum())
        groups = int((sizes > 0).sum())
    flops = 2.0 * rows * n * k
    byts = rows * k + groups * n * k + 4 * rows * kb + 4 * groups * nb * kb + rows * n * out_b
    return flops, byts


class Case:
    """One GEMM call with its inputs uploaded to the GPU."""

    def __init__(self, desc: dict, dev: str):
        import numpy as np
        import torch
        import moe_grouped_gemm_tiles_amd as dg

        self.label = desc["label"]
        self.config = desc.get("config")
        self.x = x = desc["gen"]()
        self.flops, self.bytes = algorithmic_work(x)

        def up(v):
            return torch.from_numpy(np.ascontiguousarray(v)).to(dev)

        if x["kind"] == "mqa":
            q = up(x["q"]).view(torch.float8_e4m3fn)
            kv = up(x["kv"]).view(torch.float8_e4m3fn)
            sf, w, ks, ke = up(x["sf"]), up(x["w"]), up(x["ks"]), up(x["ke"])
            out = torch.empty(x["s"], x["s_kv"], dtype=torch.float32, device=dev)
            self.call = lambda: dg.fp8_mqa_logits(q, (kv, sf), w, ks, ke, True, out)
            self.d = out
            rt_mfma = self.flops / (PEAK_FP8_TFLOPS * 1e12)
            rt_hbm = self.bytes / (PEAK_HBM_GBS * 1e9)
            self.bound = "mfma" if rt_mfma >= rt_hbm else "hbm"
            self.roof_s = max(rt_mfma, rt_hbm)
            return
        if x["kind"] in ("quant_token", "quant_block"):
            xin = up(x["x"]).to(torch.bfloat16 if x["dtype"] == "bf16" else torch.float32)
            m, k = x["m"], x["k"]
            q = torch.empty(m, k, dtype=torch.uint8, device=dev)
            if x["kind"] == "quant_token":
                sf = torch.empty(k // 128, _cdiv(m, 4) * 4, dtype=torch.float32, device=dev)
                self.call = lambda: dg.per_token_cast_to_fp8(xin, q, sf)
            else:
                sf = torch.empty(_cdiv(m, 128), k // 128, dtype=torch.float32, device=dev)
                self.call = lambda: dg.per_block_cast_to_fp8(xin, q, sf)
            self.d = q
            self.bound = "hbm"
            self.roof_s = self.bytes / (PEAK_HBM_GBS * 1e9)
            return

        a = up(x["a"]).view(torch.float8_e4m3fn)
        b = up(x["b"]).view(torch.float8_e4m3fn)
        sfa, sfb = up(x["sfa"]), up(x["sfb"])
        dt = torch.bfloat16 if x.get("out_dtype", "fp32") == "bf16" else torch.float32
        if x["kind"] == "k_grouped":
            d = torch.empty(x["num_groups"], x["m"], x["n"], dtype=torch.float32, device=dev)
            c = up(x["c"]) if x.get("c") is not None else None
            ks = up(x["ks"])
            self.call = lambda: dg.k_grouped_fp8_gemm_nt_contiguous((a, sfa), (b, sfb), d, ks, c)
        elif x["kind"] == "dense":
            d = torch.empty(x["m"], x["n"], dtype=dt, device=dev)
            c = up(x["c"]).to(dt) if x.get("c") is not None else None
            ws = dg.alloc_workspace(x["m"], x["n"], x["k"], dev)  # kept by the caller, cleared once
            self.call = lambda: dg.fp8_gemm_nt((a, sfa), (b, sfb), d, c, workspace=ws)
        elif x["kind"] == "contiguous":
            d = torch.empty(x["m_total"], x["n"], dtype=dt, device=dev)
            mi = up(x["m_indices"])
            self.call = lambda: dg.m_grouped_fp8_gemm_nt_contiguous((a, sfa), (b, sfb), d, mi)
        else:
            d = torch.empty(x["num_groups"], x["m_max"], x["n"], dtype=dt, device=dev)
            mm = up(x["masked_m"])
            em = int(x["m_max"] // 2)
            self.call = lambda: dg.m_grouped_fp8_gemm_nt_masked((a, sfa), (b, sfb), d, mm, em)
        self.d = d
        rt_mfma = self.flops / (PEAK_FP8_TFLOPS * 1e12)
        rt_hbm = self.bytes / (PEAK_HBM_GBS * 1e9)
        self.bound = "mfma" if rt_mfma >= rt_hbm else "hbm"
        self.roof_s = max(rt_mfma, rt_hbm)



class _VendorFp8:
    """The platform's FP8 GEMM on a dense case's operands (per-tensor unit scales,
    BF16 out): the same product of the E4M3 codes, without any block scaling."""

    def __init__(self, x: dict, dev: str):
        import numpy as np
        import torch

        self.a = torch.from_numpy(np.ascontiguousarray(x["a"])).to(dev).view(torch.float8_e4m3fn)
        self.b = torch.from_numpy(np.ascontiguousarray(x["b"])).to(dev).view(torch.float8_e4m3fn)
        self.one = torch.ones((), dtype=torch.float32, device=dev)
        self.call = lambda: torch._scaled_mm(self.a, self.b.t(), scale_a=self.one, scale_b=self.one,
                                             out_dtype=torch.bfloat16)


def time_launches(case: Case, iters: int, flush=None):
    """Median per-launch time (s) with HIP events on the current stream (the
    stream the library launches on)."""
    import torch
    times = []
    for _ in range(iters):
        if flush is not None:
            flush()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        case.call()
        e.record()
        e.synchronize()
        times.append(s.elapsed_time(e) * 1e-3)
    times.sort()
    return times[len(times) // 2]


def cpu_baseline(inputs, budget_rows=4096, budget_cols=24576, quant_rows=8192):
    """Time the oracle on a bounded sample of the step's inputs.

    GEMMs: the first ``budget_rows`` output rows (masked: the first two groups;
    K-grouped: every group) x the first ``budget_cols`` columns of every case,
    which is the whole step for the dense sweep; MQA: every query; casts: the
    first ``quant_rows`` rows.  Returns TFLOPS (or GB/s for the casts) of the
    oracle on the host's cores."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    total_flops, total_bytes, total_s = 0.0, 0.0, 0.0
    parts = []
    for x in inputs:
        kind = x["kind"]
        t0 = time.perf_counter()
        if kind == "mqa":
            oracle.ref_mqa_logits(x["q"], x["kv"], x["sf"], x["w"], x["ks"], x["ke"], True)
            lo = np.clip(x["ks"], 0, x["s_kv"])
            hi = np.clip(x["ke"], 0, x["s_kv"])
            total_flops += 2.0 * x["h"] * x["d"] * float(np.maximum(hi - lo, 0).sum())
            parts.append(f"all {x['s']} queries")
        elif kind in ("quant_token", "quant_block"):
            nrows = min(x["m"], quant_rows)
            (oracle.quant_per_token if kind == "quant_token" else oracle.quant_per_block)(x["x"][:nrows])
            total_bytes += nrows * x["k"] * (2 if x["dtype"] == "bf16" else 4) + nrows * x["k"]
            parts.append(f"{nrows} of {x['m']} rows")
        else:
            n, k = x["n"], x["k"]
            cols = np.arange(min(n, budget_cols))
            ue = x.get("scale_fmt") == "ue8m0"
            if kind == "k_grouped":
                rows = np.arange(min(x["m"], budget_rows))
                ref = oracle.ref_k_grouped_ue8m0 if ue else oracle.ref_k_grouped
                ref(x["a"], x["sfa"], x["b"], x["sfb"], x["ks"], x.get("c"), rows=rows, cols=cols)
                nrows = len(rows)
            elif kind == "dense":
                rows = np.arange(min(x["m"], budget_rows))
                ref = oracle.ref_dense_ue8m0 if ue else oracle.ref_dense
                ref(x["a"], x["sfa"], x["b"], x["sfb"], x.get("c"), rows=rows, cols=cols)
                nrows = len(rows)
            elif kind == "contiguous":
                valid = np.nonzero(x["m_indices"] >= 0)[0][:budget_rows]
                ref = oracle.ref_contiguous_ue8m0 if ue else oracle.ref_contiguous
                ref(x["a"], x["sfa"], x["b"], x["sfb"], x["m_indices"], rows=valid, cols=cols)
                nrows = len(valid)
            else:
                groups = np.arange(min(x["num_groups"], 2))
                ref = oracle.ref_masked_ue8m0 if ue else oracle.ref_masked
                ref(x["a"], x["sfa"], x["b"], x["sfb"], x["masked_m"], groups=groups, cols=cols)
                nrows = int(np.clip(x["masked_m"][groups], 0, x["m_max"]).sum())
            total_flops += 2.0 * nrows * len(cols) * k
            parts.append(f"{nrows} rows x {len(cols)} cols")
        total_s += time.perf_counter() - t0
    host = len(os.sched_getaffinity(0))
    if total_flops == 0:
        return dict(value=total_bytes / total_s / 1e9, unit="GB/s", cores=int(threads), kind="oracle",
                    sample=f"numpy FP32 cast of {'; '.join(parts)}: {total_bytes / 1e6:.1f} MB in {total_s:.1f} s",
                    host_cpus=host)
    return dict(value=total_flops / total_s / 1e12, unit="TFLOPS", cores=int(threads), kind="oracle",
                sample=f"FP64 numpy oracle over {'; '.join(parts)} of the step's cases: "
                       f"{total_flops / 1e9:.1f} GFLOP in {total_s:.1f} s",
                host_cpus=host)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="baseline")
    ap.add_argument("--cases", default="", help="comma-separated case indices of the workload to keep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush-mb", type=int, default=512, help="cache flush buffer for the per-shape cold timing")
    ap.add_argument("--timing-iters", type=int, default=10, help="launches per shape for the warm/cold timing")
    ap.add_argument("--vendor-fp8", action="store_true",
                    help="also time the platform's per-tensor-scaled FP8 GEMM (torch._scaled_mm) on each dense "
                         "case's operands, as context (it skips the block scaling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help=f"run one {COPY_CAL_MB} MiB device copy first (calibrates rocprofv3 byte counters)")
    ap.add_argument("--profile-summary", nargs=3, metavar=("PROF_DIR", "OUT_MD", "CASE_LABEL"),
                    help="summarise rocprofv3 output collected for CASE_LABEL and exit (no GPU needed)")
    ap.add_argument("--profile-command", default="", help="command line recorded in the profile summary")
    ap.add_argument("--profile-kernel", default="gemm_kernel", help="name substring of the profiled kernel")
    ap.add_argument("--counter-summary", nargs=5, metavar=("PROF_DIR", "OUT_MD", "CASE_LABEL", "FLOPS", "LAUNCH_US"),
                    help="summarise rocprofv3 --pmc counter runs for CASE_LABEL and exit (no GPU needed)")
    args = ap.parse_args()

    if args.profile_summary:
        profile_summary(*args.profile_summary, command=args.profile_command, kernel=args.profile_kernel)
        return
    if args.counter_summary:
        d, out, label, flops, us = args.counter_summary
        counter_summary(d, out, label, args.profile_command, args.profile_kernel, float(flops), float(us))
        return

    if args.gpus != 1:
        print("bench.py: this library is measured on one GPU; --gpus above 1 is not supported "
              "(multi-GPU sharding is a design note only).", file=sys.stderr)
        sys.exit(2)

    import torch
    from workloads import workload

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.ones(COPY_CAL_MB * (1 << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    descs = workload(args.workload)
    if args.cases:
        keep = [int(v) for v in args.cases.split(",")]
        descs = [descs[i] for i in keep]
    print(f"bench: generating {len(descs)} case(s) of {args.workload}", file=sys.stderr, flush=True)
    cases = []
    for desc in descs:
        c = Case(desc, dev)
        cases.append(c)
        print(f"bench:   {c.label}: {c.flops / 1e9:.1f} GFLOP, {c.bytes / 1e6:.1f} MB, {c.bound}-bound",
              file=sys.stderr, flush=True)

    # per-launch timing, warm (back to back) and cold (after a cache flush).
    # Cold is the kernel's own time: the flush keeps the GPU busy while the
    # host enqueues the launch, so no host gap lands between the events.
    # read-only flush: evicts the operands from L2 and the Infinity Cache without
    # leaving dirty lines whose write-back would overlap the timed launch
    flush_buf = torch.ones(args.flush_mb * (1 << 20) // 4, dtype=torch.float32, device=dev)
    flush = lambda: flush_buf.sum()
    detail = []
    for c in cases:
        c.call()
        torch.cuda.synchronize()
        warm = time_launches(c, args.timing_iters)
        cold = time_launches(c, args.timing_iters, flush)
        c.warm_s, c.cold_s = warm, cold
        detail.append(dict(case=c.label, config=c.config, bound=c.bound, tflops_cold=c.flops / cold / 1e12,
                           tflops_warm=c.flops / warm / 1e12, us_cold=cold * 1e6, us_warm=warm * 1e6,
                           roofline_frac_cold=c.roof_s / cold, roofline_frac_warm=c.roof_s / warm))
        print(f"bench:   {c.label}: cold {cold * 1e6:.1f} us ({c.flops / cold / 1e12:.1f} TFLOPS, "
              f"{100 * c.roof_s / cold:.1f}% of roofline), warm {warm * 1e6:.1f} us", file=sys.stderr, flush=True)
        if args.vendor_fp8 and c.x["kind"] == "dense" and c.x.get("c") is None:
            v = _VendorFp8(c.x, dev)
            v.call()
            torch.cuda.synchronize()
            v_warm, v_cold = time_launches(v, args.timing_iters), time_launches(v, args.timing_iters, flush)
            detail[-1].update(vendor_fp8_us_cold=v_cold * 1e6, vendor_fp8_us_warm=v_warm * 1e6,
                              vendor_fp8_tflops_cold=c.flops / v_cold / 1e12)
            print(f"bench:     per-tensor FP8 torch._scaled_mm, same operands: cold {v_cold * 1e6:.1f} us "
                  f"({c.flops / v_cold / 1e12:.1f} TFLOPS), warm {v_warm * 1e6:.1f} us", file=sys.stderr, flush=True)
            del v
    # the floor under every cold time: a minimal library call (M=1, N=16, K=128,
    # 32 KFLOP) timed the same way, cold and warm
    floor = None
    if cases[0].x["kind"] in ("dense", "contiguous", "masked", "k_grouped"):
        from workloads import gen_dense
        tiny = Case(dict(label="floor", gen=lambda: gen_dense(1, 16, 128, seed=9)), dev)
        tiny.call()
        torch.cuda.synchronize()
        floor = dict(us_cold=time_launches(tiny, args.timing_iters, flush) * 1e6,
                     us_warm=time_launches(tiny, args.timing_iters) * 1e6,
                     what="dense M=1 N=16 K=128 through the same entry point, timed like the cases")
        print(f"bench:   launch floor: cold {floor['us_cold']:.1f} us, warm {floor['us_warm']:.1f} us",
              file=sys.stderr, flush=True)
    del flush_buf
    dom = max(range(len(cases)), key=lambda i: cases[i].warm_s)

    # the timed steps (the dominant case bracketed by HIP events on the launch stream)
    for _ in range(args.warmup):
        for c in cases:
            c.call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    marks = _RangeMarks()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for i, c in enumerate(cases):
            if i == dom:
                marks.push(TIMED_MARK + c.label)
                ev[s][0].record()
                c.call()
                ev[s][1].record()
                marks.pop()
            else:
                c.call()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    dom_s = sum(a.elapsed_time(b) for a, b in ev) * 1e-3 / args.steps
    step_flops = sum(c.flops for c in cases)
    step_bytes = sum(c.bytes for c in cases)
    if step_flops > 0 and cases[0].x["kind"] == "mqa":
        metric = "FP8 MQA-logits TFLOPS (2*H*D per valid query-key pair) and % of MI355X dense-FP8 peak"
        value, unit = step_flops * args.steps / elapsed / 1e12, "TFLOPS"
    elif step_flops > 0:
        metric = "FP8 scaled-GEMM TFLOPS and % of MI355X dense-FP8 peak (dense, grouped)"
        value, unit = step_flops * args.steps / elapsed / 1e12, "TFLOPS"
    else:
        metric = "FP8 cast throughput, GB/s of algorithmic HBM traffic (read input + write codes and scales)"
        value, unit = step_bytes * args.steps / elapsed / 1e9, "GB/s"

    dc = cases[dom]
    if dc.bound == "mfma":
        roof = dict(bound="mfma", achieved=dc.flops / dom_s / 1e12, peak=PEAK_FP8_TFLOPS, unit="TFLOP/s")
    else:
        roof = dict(bound="hbm", achieved=dc.bytes / dom_s / 1e9, peak=PEAK_HBM_GBS, unit="GB/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = lookup_traffic(dc.label)
    roof["kernel_case"] = dc.label
    roof["avg_launch_us"] = dom_s * 1e6

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline([c.x for c in cases])

    out = {
        "metric": metric,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 x fp8_e4m3 -> fp32 accumulate" if step_flops > 0 else "bf16 -> fp8_e4m3 + fp32 scales",
        "data": "synthetic (seeded N(0,1) q and kv cast to E4M3, kv scaled per row by amax/448, "
                "weights N(0,1)/sqrt(H), causal ranges)" if cases[0].x["kind"] == "mqa" else
                ("synthetic (seeded N(0,1), quantized to E4M3 with 1x128 / 128x128 "
                 + ("UE8M0 power-of-two" if cases[0].x.get("scale_fmt") == "ue8m0" else "FP32") + " scales)")
                if step_flops > 0 else "synthetic (seeded N(0,1) rows with e^U(-4,4) magnitude spread, BF16)",
        "config": {"workload": args.workload, "cases": [c.label for c in cases],
                   "out_dtype": sorted({c.x.get("out_dtype", "fp32") for c in cases if "out_dtype" in c.x})},
        "roofline": roof,
        "cpu_baseline": cpu,
        "detail": detail,
        "launch_floor": floor,
    }
    if step_flops > 0:
        out["config"]["pct_of_fp8_peak"] = 100.0 * value / PEAK_FP8_TFLOPS
    groups = {}
    for c in cases:
        if c.config is not None:
            groups.setdefault(c.config, []).append(c)
    if groups:
        out["config"]["configs"] = {str(g): [c.label for c in cs] for g, cs in sorted(groups.items())}
        summ = {}
        for g, cs in sorted(groups.items()):
            fl = sum(c.flops for c in cs)
            cold = sum(c.cold_s for c in cs)
            roof = sum(c.roof_s for c in cs)
            summ[str(g)] = dict(cases=len(cs), tflops_cold=fl / cold / 1e12, us_cold=cold * 1e6,
                                roofline_frac_cold=roof / cold,
                                bound="+".join(sorted({c.bound for c in cs})))
        out["summary_by_config"] = summ
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
