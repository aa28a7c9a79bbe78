"""HIP-graph capture of library calls.

The library allocates nothing and never synchronises, so every entry point can
be captured, also as the first call of its shape.  Graphs are replayed several
times with eager work and synchronisations between replays, and every replay
must reproduce the eager outputs bit for bit, including the rows the library
must leave unwritten.
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
        ws = dg.alloc_workspace(x["m"], x["n"], x["k"])
        out.append((name, (lambda a=a, b=b, sfa=sfa, sfb=sfb, d=d, c=c, ws=ws:
                           dg.fp8_gemm_nt((a, sfa), (b, sfb), d, c, workspace=ws)), d))
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


def test_split_k_captured_first_and_replayed_on_another_stream():
    """Skinny (split-K) calls captured with no eager call of their shape before, one with
    a caller workspace and one with the per-call workspace the binding takes from torch
    (allocated and cleared inside the capture); replays alternate between the capture
    stream and a second stream and must equal eager calls made afterwards."""
    xs = [gen_dense(64, 2112, 7168, seed=190), gen_dense(100, 1040, 4096, seed=191, with_c=True),
          gen_dense(128, 24576, 1536, seed=192)]
    dev = []
    for x in xs:
        c = to_dev(x["c"]).to(torch.bfloat16) if x["c"] is not None else None
        dev.append((fp8_dev(x["a"]), to_dev(x["sfa"]), fp8_dev(x["b"]), to_dev(x["sfb"]), c,
                    torch.empty(x["m"], x["n"], dtype=torch.bfloat16, device="cuda:0")))
    ws0 = dg.alloc_workspace(64, 2112, 7168)
    ws2 = dg.alloc_workspace(128, 24576, 1536)
    wss = [ws0, None, ws2]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s1):
        for (a, sfa, b, sfb, c, d), ws in zip(dev, wss):
            dg.fp8_gemm_nt((a, sfa), (b, sfb), d, c, workspace=ws)
    torch.cuda.synchronize()
    want = []
    for a, sfa, b, sfb, c, d in dev:  # eager, each with a fresh workspace
        e = torch.empty_like(d)
        dg.fp8_gemm_nt((a, sfa), (b, sfb), e, c)
        want.append(e)
    torch.cuda.synchronize()
    want = [_bits(e) for e in want]
    scratch = torch.randn(1 << 20, device="cuda:0")
    for r in range(6):
        for *_, d in dev:
            _sentinel_fill(d)
        scratch.mul_(1.0001).add_(0.5)
        torch.cuda.synchronize()
        with torch.cuda.stream(s2 if r % 2 else s1):
            g.replay()
        torch.cuda.synchronize()
        for i, (*_, d) in enumerate(dev):
            assert torch.equal(_bits(d), want[i]), f"replay {r}: call {i} differs from the eager result"
        note(f"replay {r} on stream {2 if r % 2 else 1}: split-K outputs bit-identical to eager")
