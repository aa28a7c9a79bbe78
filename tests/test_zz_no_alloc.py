"""The allocation-free dense entry point (dg_fp8_gemm_nt_noalloc), called through
the C ABI, against the workspace entry point (dg_fp8_gemm_nt) on the same inputs:
bit-identical outputs (same kernels and split counts) and within the oracle's
tolerance, on consecutive calls whose second input is smaller, with and without C,
for a shape that does not split K, and captured into a HIP graph that is replayed
after eager calls of another shape have used the same scratch.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import gen_dense

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():  # pragma: no cover - GPU only
    import moe_grouped_gemm_tiles_amd as dg
    from tests._gpu_harness import SENT_BF16, SENT_F32, as_f64, c_tensor, fp8_dev, note, out_buffer, raw_bits, to_dev


def _args(x, d, c=None):
    a, sfa, b, sfb = fp8_dev(x["a"]), to_dev(x["sfa"]), fp8_dev(x["b"]), to_dev(x["sfb"])
    es = d.element_size()
    keep = (a, sfa, b, sfb, c)
    args = (a.data_ptr(), a.stride(0), sfa.data_ptr(), sfa.stride(0), b.data_ptr(), b.stride(0), sfb.data_ptr(),
            c.data_ptr() if c is not None else None, c.stride(0) if c is not None else 0, d.data_ptr(), d.stride(0),
            0 if d.dtype == torch.bfloat16 else 1, x["m"], x["n"], x["k"])
    return keep, args


def _with_workspace(x, d, c=None):
    lib = dg.load_library()
    keep, args = _args(x, d, c)
    ws = dg.alloc_workspace(x["m"], x["n"], x["k"])
    st = lib.dg_fp8_gemm_nt(*args, ws.data_ptr() if ws is not None else None,
                            ws.numel() if ws is not None else 0, torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.dg_status_string(st)
    torch.cuda.synchronize()


def _noalloc(x, d, c=None):
    lib = dg.load_library()
    keep, args = _args(x, d, c)
    st = lib.dg_fp8_gemm_nt_noalloc(*args, torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.dg_status_string(st)
    torch.cuda.synchronize()


@pytest.mark.parametrize("with_c", [False, True])
def test_noalloc_matches_workspace_entry_point_on_two_calls(with_c):
    # the second call is smaller (fewer tiles, fewer splits) and reuses the same scratch
    for m, n, k, seed in ((128, 7168, 16384, 1500), (64, 2112, 7168, 1501)):
        out = "fp32" if with_c else "bf16"
        x = gen_dense(m, n, k, seed=seed + with_c, with_c=with_c, out_dtype=out)
        assert dg.get_workspace_size(m, n, k) > 0
        c = c_tensor(x["c"], out) if with_c else None
        want = out_buffer((m,), n, out)
        _with_workspace(x, want, c)
        got = out_buffer((m,), n, out)
        _noalloc(x, got, c)
        assert np.array_equal(raw_bits(got), raw_bits(want)), f"M={m} N={n} K={k}: differs from dg_fp8_gemm_nt"
        ref = oracle.ref_dense(x["a"], x["sfa"], x["b"], x["sfb"], x["c"])
        rep = oracle.assert_close(as_f64(got), ref, f"noalloc M={m} N={n} K={k} C={with_c}")
        note(f"noalloc M={m} N={n} K={k} C={with_c}: bit-identical, worst={rep['worst_ratio']:.3f}")


def test_noalloc_repeated_and_unsplit_shapes():
    xs = [gen_dense(100, 1040, 4096, seed=1510), gen_dense(300, 520, 1024, seed=1511),
          gen_dense(1, 300 * 8, 2048, seed=1512)]
    want = []
    for x in xs:
        d = out_buffer((x["m"],), x["n"], "bf16")
        _with_workspace(x, d)
        want.append(raw_bits(d))
    for rep in range(3):
        for i, x in enumerate(xs):
            d = out_buffer((x["m"],), x["n"], "bf16")
            _noalloc(x, d)
            assert np.array_equal(raw_bits(d), want[i]), f"repeat {rep}, input {i}"


def _noalloc_launch(args):
    """One call on the current stream, no synchronisation (capturable)."""
    lib = dg.load_library()
    st = lib.dg_fp8_gemm_nt_noalloc(*args, torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.dg_status_string(st)


def test_noalloc_captured_in_a_graph_and_replayed():
    """The callers this entry point serves capture it: one graph holds two split-K calls
    of different shapes (the second smaller, with C); before every replay an eager call
    of a third shape leaves its own partials and counters in the shared scratch, and
    every replay must still equal the workspace entry point bit for bit."""
    calls = []
    for (m, n, k), with_c, seed in (((128, 2112, 7168), False, 1520), ((64, 1040, 4096), True, 1521)):
        assert dg.get_workspace_size(m, n, k) > 0  # K is split: the call uses the scratch
        out = "fp32" if with_c else "bf16"
        x = gen_dense(m, n, k, seed=seed, with_c=with_c, out_dtype=out)
        c = c_tensor(x["c"], out) if with_c else None
        want = out_buffer((m,), n, out)
        _with_workspace(x, want, c)
        d = out_buffer((m,), n, out)
        keep, args = _args(x, d, c)
        calls.append((f"M={m} N={n} K={k}", d, keep, args, raw_bits(want)))
    other = gen_dense(100, 520, 8192, seed=1522)
    assert dg.get_workspace_size(100, 520, 8192) > 0
    other_d = out_buffer((100,), 520, "bf16")
    other_want = out_buffer((100,), 520, "bf16")
    _with_workspace(other, other_want)
    _noalloc(other, other_d)  # the scratch address is looked up on an eager call, not under capture
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for *_, args, _ in calls:
            _noalloc_launch(args)
    torch.cuda.synchronize()
    for r in range(4):
        _noalloc(other, other_d)  # eager, same scratch, another tile grid and split count
        assert np.array_equal(raw_bits(other_d), raw_bits(other_want)), f"eager call before replay {r}"
        for _, d, _, _, _ in calls:
            if d.dtype == torch.bfloat16:
                d.view(torch.int16).fill_(SENT_BF16)
            else:
                d.view(torch.int32).fill_(SENT_F32)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        for name, d, _, _, want in calls:
            assert np.array_equal(raw_bits(d), want), f"replay {r}: {name} differs from dg_fp8_gemm_nt"
        note(f"noalloc graph replay {r}: both captured calls bit-identical")
