"""HIP-graph capture of library calls (the benchmark times graph replays).

The calls are captured on one stream after an eager run on that stream (which
creates any split-K workspace, so nothing is allocated during capture).  The
graph is replayed several times with eager work and synchronisations between
replays, and every replay must reproduce the eager outputs bit for bit,
including the rows the library must leave unwritten.
"""

import numpy as np
import pytest
import torch

from workloads import gen_contiguous, gen_dense, gen_k_grouped, gen_masked

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():  # pragma: no cover - GPU only
    import moe_grouped_gemm_tiles_amd as dg
    from tests._gpu_harness import SENT_BF16, SENT_F32, fp8_dev, note, to_dev


def _sentinel_fill(d):
    if d.dtype == torch.bfloat16:
        d.view(torch.int16).fill_(SENT_BF16)
    else:
        d.view(torch.int32).fill_(SENT_F32)


def _bits(d):
    return d.view(torch.int16 if d.dtype == torch.bfloat16 else torch.int32).clone()


def _calls():
    """(name, call, output) for one call of every kernel family."""
    out = []
    for name, x in (("dense 256x256", gen_dense(512, 1024, 1024, seed=90)),
                    ("dense split-K", gen_dense(64, 2112, 2048, seed=91)),
                    ("dense split-K + C", gen_dense(100, 520, 2048, seed=92, with_c=True, out_dtype="fp32")),
                    ("dense ue8m0", gen_dense(300, 400, 1152, seed=93, scale_fmt="ue8m0"))):
        a, b, sfa, sfb = fp8_dev(x["a"]), fp8_dev(x["b"]), to_dev(x["sfa"]), to_dev(x["sfb"])
        dt = torch.bfloat16 if x["out_dtype"] == "bf16" else torch.float32
        d = torch.empty(x["m"], x["n"], dtype=dt, device="cuda:0")
        c = to_dev(x["c"]).to(dt) if x["c"] is not None else None
        out.append((name, (lambda a=a, b=b, sfa=sfa, sfb=sfb, d=d, c=c: dg.fp8_gemm_nt((a, sfa), (b, sfb), d, c)), d))
    x = gen_contiguous(3, 384, 512, seed=94, m_sizes=[130, 0, 200])
    d = torch.empty(x["m_total"], 384, dtype=torch.bfloat16, device="cuda:0")
    args = ((fp8_dev(x["a"]), to_dev(x["sfa"])), (fp8_dev(x["b"]), to_dev(x["sfb"])), d, to_dev(x["m_indices"]))
    out.append(("contiguous", (lambda args=args: dg.m_grouped_fp8_gemm_nt_contiguous(*args)), d))
    x = gen_masked(4, 256, 512, 1024, seed=95, masked_m=[0, 256, 31, 200])
    d = torch.empty(4, 256, 512, dtype=torch.bfloat16, device="cuda:0")
    args = ((fp8_dev(x["a"]), to_dev(x["sfa"])), (fp8_dev(x["b"]), to_dev(x["sfb"])), d, to_dev(x["masked_m"]), 200)
    out.append(("masked", (lambda args=args: dg.m_grouped_fp8_gemm_nt_masked(*args)), d))
    x = gen_k_grouped(3, 256, 384, seed=96, ks=[512, 0, 256])
    d = torch.empty(3, 256, 384, dtype=torch.float32, device="cuda:0")
    args = ((fp8_dev(x["a"]), to_dev(x["sfa"])), (fp8_dev(x["b"]), to_dev(x["sfb"])), d, to_dev(x["ks"]),
            to_dev(x["c"]))
    out.append(("k-grouped", (lambda args=args: dg.k_grouped_fp8_gemm_nt_contiguous(*args)), d))
    x = gen_k_grouped(3, 256, 384, seed=97, ks=[128, 384, 0], scale_fmt="ue8m0")
    d = torch.empty(3, 256, 384, dtype=torch.float32, device="cuda:0")
    args = ((fp8_dev(x["a"]), to_dev(x["sfa"])), (fp8_dev(x["b"]), to_dev(x["sfb"])), d, to_dev(x["ks"]),
            to_dev(x["c"]))
    out.append(("k-grouped ue8m0", (lambda args=args: dg.k_grouped_fp8_gemm_nt_contiguous(*args)), d))
    sf = to_dev(np.exp2(np.random.default_rng(98).integers(-8, 8, (2, 70, 9))).astype(np.float32))
    d = torch.empty(2, 3, 72, dtype=torch.int32, device="cuda:0")
    lib = dg.load_library()

    def layout(sf=sf, d=d):
        st = lib.dg_transform_sf_into_required_layout(sf.data_ptr(), d.data_ptr(), 2, 70, 9, 72, 1,
                                                      torch.cuda.current_stream().cuda_stream)
        assert st == 0

    out.append(("scale layout ue8m0", layout, d))
    return out


def test_graph_replays_match_eager():
    calls = _calls()
    s = torch.cuda.Stream()
    ref = []
    with torch.cuda.stream(s):
        for name, fn, d in calls:
            _sentinel_fill(d)
            fn()
    torch.cuda.synchronize()
    ref = [_bits(d) for _, _, d in calls]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _, fn, _ in calls:
            fn()
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda:0")
    for r in range(4):
        for _, _, d in calls:
            _sentinel_fill(d)  # eager work between replays
        scratch.mul_(1.0001).add_(0.5)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        for (name, _, d), want in zip(calls, ref):
            assert torch.equal(_bits(d), want), f"replay {r}: {name} differs from the eager result"
        note(f"replay {r}: all {len(calls)} outputs bit-identical to eager")
