"""GPU tests of the skinny dense path (M <= 128): K split across workgroups in
one launch, partials in a caller-owned workspace, the last workgroup of each
tile adding them in K-range order.  Checked against the FP64 oracle, for
determinism, for workspace reuse across shapes and for the workspace errors of
the C ABI; plus the BF16-with-C column edge and the masked scale-row length.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from workloads import gen_dense, gen_masked

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():  # pragma: no cover - GPU only
    import moe_grouped_gemm_tiles_amd as dg
    from tests._gpu_harness import (as_f64, c_tensor, fp8_dev, note, out_buffer, raw_bits, run_dense,
                                    sentinel_of, to_dev)

DG_ERROR_WORKSPACE = 4


def _dev_inputs(x):
    return fp8_dev(x["a"]), to_dev(x["sfa"]), fp8_dev(x["b"]), to_dev(x["sfb"])


def _call(x, d, ws=None, c=None):
    a, sfa, b, sfb = _dev_inputs(x)
    dg.fp8_gemm_nt((a, sfa), (b, sfb), d, c, workspace=ws)


@pytest.mark.parametrize("m,n,k", [(1, 2112, 7168), (64, 2112, 7168), (64, 7168, 2048), (100, 1040, 4096),
                                   (128, 4096, 7168), (128, 24576, 1536), (33, 300, 512), (128, 200, 640)])
def test_split_k_shapes(m, n, k):
    """Skinny shapes, split or not as the dispatcher decides (many tiles: no split)."""
    x = gen_dense(m, n, k, seed=1000 + m + n + k)
    d = run_dense(x, ld_d=(n + 7) // 8 * 8 + 8)
    ref = oracle.ref_dense(x["a"], x["sfa"], x["b"], x["sfb"])
    rep = oracle.assert_close(as_f64(d), ref, f"split-K M={m} N={n} K={k}")
    note(f"split-K M={m} N={n} K={k}: worst={rep['worst_ratio']:.3f} ws={dg.get_workspace_size(m, n, k)} B")


@pytest.mark.parametrize("m,out", [(48, "fp32"), (128, "bf16"), (100, "fp32"), (64, "bf16")])
def test_split_k_with_c_and_in_place(m, out):
    x = gen_dense(m, 1005 if out == "bf16" else 520, 2048, seed=60 + m, with_c=True, out_dtype=out)
    ref = oracle.ref_dense(x["a"], x["sfa"], x["b"], x["sfb"], x["c"])
    d = run_dense(x, ld_d=1024)
    oracle.assert_close(as_f64(d), ref, f"split-K + C M={m} {out}")
    d2 = run_dense(x, ld_d=1024, c_in_place=True)
    oracle.assert_close(as_f64(d2), ref, f"split-K + C in place M={m} {out}")
    assert np.array_equal(raw_bits(d), raw_bits(d2))


def test_wgrad_split_k_in_place():
    x = gen_dense(64, 384, 4096, seed=62, with_c=True, out_dtype="fp32")
    a, sfa, b, sfb = _dev_inputs(x)
    d = to_dev(x["c"].astype(np.float32))
    dg.wgrad_fp8_gemm_nt((a, sfa), (b, sfb), d, workspace=dg.alloc_workspace(64, 384, 4096))
    torch.cuda.synchronize()
    oracle.assert_close(as_f64(d), oracle.ref_dense(x["a"], x["sfa"], x["b"], x["sfb"], x["c"]), "wgrad split-K")


def test_small_shapes_split():
    for m, n, k in ((1, 2112, 7168), (64, 2112, 7168), (64, 7168, 2048), (100, 1040, 4096), (128, 4096, 7168),
                    (128, 7168, 16384)):
        assert dg.get_workspace_size(m, n, k) > 0, f"M={m} N={n} K={k} expected to split K"
    assert dg.get_workspace_size(129, 4096, 7168) == 0  # M > 128: no split


@pytest.mark.parametrize("m,n,k,cap,out,with_c,in_place", [
    (128, 1005, 8192, 32, "bf16", True, False), (100, 520, 8192, 24, "fp32", True, True),
    (96, 1005, 4096, 32, "bf16", False, False), (128, 520, 4096, 16, "fp32", False, False),
    (128, 1005, 8192, 48, "fp32", True, False)])
def test_128_column_split_tile(m, n, k, cap, out, with_c, in_place):
    """64 < M <= 128 on a CU cap where the planner takes 128x128 tiles with K split:
    D (with or without C, in place or not) against the oracle, columns past N untouched."""
    plan = dg._dense_plan_for_tests(m, n, k, cap)
    assert (plan["bm"], plan["bn"]) == (128, 128) and plan["splits"] > 1, plan
    note(f"128x128 split M={m} N={n} K={k} cap={cap} {out} C={with_c} in_place={in_place}: {plan}")
    x = gen_dense(m, n, k, seed=7 * m + n + k, with_c=with_c, out_dtype=out)
    ref = oracle.ref_dense(x["a"], x["sfa"], x["b"], x["sfb"], x.get("c"))
    try:
        dg.set_num_cus(cap)
        assert dg.get_workspace_size(m, n, k) == plan["ws_bytes"]
        d = run_dense(x, ld_d=1024, c_in_place=in_place)
        d2 = run_dense(x, ld_d=1024, c_in_place=in_place)
    finally:
        dg.set_num_cus(0)
    oracle.assert_close(as_f64(d), ref, f"128x128 split M={m} N={n} K={k}")
    assert np.array_equal(raw_bits(d), raw_bits(d2)), "not deterministic"
    full = d.as_strided((m, 1024), (1024, 1))
    pad = 0 if in_place else sentinel_of(d)  # C's padding is zero-filled
    assert (raw_bits(full)[:, n:] == pad).all(), "columns past N were written"


def test_one_workspace_serves_a_sequence_of_shapes():
    """Calls of different shapes share one zero-filled workspace on one stream; each
    leaves the counters at zero, so every output equals the result with a fresh workspace."""
    shapes = [(64, 2112, 7168), (128, 24576, 1536), (1, 7168, 2048), (100, 1040, 4096), (64, 2112, 7168),
              (128, 4096, 7168), (33, 300, 512)]
    xs = [gen_dense(m, n, k, seed=1100 + i) for i, (m, n, k) in enumerate(shapes)]
    ld = [(x["n"] + 7) // 8 * 8 for x in xs]  # BF16 rows of whole 16-byte units
    want = [raw_bits(run_dense(x, ld_d=ld[i])) for i, x in enumerate(xs)]
    size = max(dg.get_workspace_size(m, n, k) for m, n, k in shapes)
    assert size > 0
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda:0")
    outs = []
    for rep in range(3):
        for i, x in enumerate(xs):
            d = out_buffer((x["m"],), x["n"], x["out_dtype"], ld[i])
            _call(x, d, ws)
            outs.append(d)
    torch.cuda.synchronize()
    for i, d in enumerate(outs):
        assert np.array_equal(raw_bits(d), want[i % len(xs)]), f"call {i} ({shapes[i % len(xs)]})"
    ctr_words = ws[:65536].view(torch.int32)
    assert not ctr_words.any(), "tile counters not reset to zero"


def test_cu_cap_changes_splits_results_agree():
    x = gen_dense(64, 2112, 7168, seed=1200)
    ref = oracle.ref_dense(x["a"], x["sfa"], x["b"], x["sfb"])
    base = dg.get_workspace_size(64, 2112, 7168)
    try:
        for cap in (7, 64, 160):
            dg.set_num_cus(cap)
            size = dg.get_workspace_size(64, 2112, 7168)
            d1, d2 = run_dense(x), run_dense(x)
            assert np.array_equal(raw_bits(d1), raw_bits(d2)), f"cap {cap}: not deterministic"
            oracle.assert_close(as_f64(d1), ref, f"split-K capped at {cap} CUs (ws {size} B)")
    finally:
        dg.set_num_cus(0)
    assert dg.get_workspace_size(64, 2112, 7168) == base


def test_workspace_errors_through_the_c_abi():
    m, n, k = 64, 2112, 7168
    x = gen_dense(m, n, k, seed=1300)
    a, sfa, b, sfb = _dev_inputs(x)
    d = out_buffer((m,), n, "bf16")
    lib = dg.load_library()
    size = lib.dg_get_workspace_size(m, n, k)
    assert size > 0
    ws = torch.zeros(size + 512, dtype=torch.uint8, device="cuda:0")
    base = ws.data_ptr() + (-ws.data_ptr()) % 256
    stream = torch.cuda.current_stream().cuda_stream

    def call(ptr, nbytes):
        return lib.dg_fp8_gemm_nt(a.data_ptr(), k, sfa.data_ptr(), sfa.stride(0), b.data_ptr(), k, sfb.data_ptr(),
                                  None, 0, d.data_ptr(), n, 0, m, n, k, ptr, nbytes, stream)

    assert call(None, 0) == DG_ERROR_WORKSPACE
    assert call(base, size - 4) == DG_ERROR_WORKSPACE
    assert call(base + 16, size) == DG_ERROR_WORKSPACE  # not 256-byte aligned
    torch.cuda.synchronize()
    assert (raw_bits(d) == sentinel_of(d)).all(), "a refused call wrote D"
    assert call(base, size) == 0
    torch.cuda.synchronize()
    oracle.assert_close(as_f64(d), oracle.ref_dense(x["a"], x["sfa"], x["b"], x["sfb"]), "C ABI with workspace")
    assert b"DG_ERROR_WORKSPACE" in lib.dg_status_string(DG_ERROR_WORKSPACE)


@pytest.mark.parametrize("m,n,k,in_place", [(300, 1005, 256, False), (300, 13, 384, True), (260, 229, 384, False),
                                            (96, 1005, 2048, True), (128, 229, 4096, False), (40, 13, 1024, True)])
def test_bf16_with_c_ragged_columns(m, n, k, in_place):
    """BF16 output plus a BF16 C with N not a multiple of 4 or 8: C's edge columns go
    through the element path; columns past N (padded leading dimension) keep the sentinel."""
    ld = (n + 7) // 8 * 8 + 8
    x = gen_dense(m, n, k, seed=5 * n + k + m, with_c=True, out_dtype="bf16")
    a, sfa, b, sfb = _dev_inputs(x)
    c = c_tensor(x["c"], "bf16", ld)
    full_c = c.as_strided((m, ld), (ld, 1))
    if in_place:
        full_c[:, n:].view(torch.int16).fill_(np.int16(0x7FBF))
        d = c
    else:
        d = out_buffer((m,), n, "bf16", ld)
    dg.fp8_gemm_nt((a, sfa), (b, sfb), d, c)
    torch.cuda.synchronize()
    c_bf16 = torch.from_numpy(x["c"].astype(np.float32)).to(torch.bfloat16).double().numpy()
    ref = oracle.ref_dense(x["a"], x["sfa"], x["b"], x["sfb"], c_bf16)
    oracle.assert_close(as_f64(d), ref, f"bf16+C ragged N m={m} n={n} k={k} in_place={in_place}")
    full = d.as_strided((m, ld), (ld, 1))
    assert (raw_bits(full)[:, n:] == sentinel_of(d)).all(), "columns past N were written"


def test_masked_one_scale_row_needs_aligned_row_length():
    """K = 128 gives one scale row per group; an sfa row length that is not a multiple
    of 4 is refused (the library steps groups by rows x row length)."""
    g, m_max, n, k = 3, 70, 256, 128
    x = gen_masked(g, m_max, n, k, seed=1400, masked_m=[70, 5, 33])
    sfa = np.ascontiguousarray(x["sfa"][:, :, :m_max])  # row length 70
    d = out_buffer((g, m_max), n, "bf16")
    with pytest.raises(RuntimeError, match="INVALID"):
        dg.m_grouped_fp8_gemm_nt_masked((fp8_dev(x["a"]), to_dev(sfa)), (fp8_dev(x["b"]), to_dev(x["sfb"])), d,
                                        to_dev(x["masked_m"]), 64)
    torch.cuda.synchronize()
    assert (raw_bits(d) == sentinel_of(d)).all()
    # the padded layout (row length 72) works, and every group reads its own scales
    d = out_buffer((g, m_max), n, "bf16")
    dg.m_grouped_fp8_gemm_nt_masked((fp8_dev(x["a"]), to_dev(x["sfa"])), (fp8_dev(x["b"]), to_dev(x["sfb"])), d,
                                    to_dev(x["masked_m"]), 64)
    torch.cuda.synchronize()
    ref, written = oracle.ref_masked(x["a"], x["sfa"], x["b"], x["sfb"], x["masked_m"])
    oracle.assert_close(as_f64(d)[written], ref[written], "masked K=128")
    assert (raw_bits(d)[~written] == sentinel_of(d)).all()


def _cap_for_128_column_split(m, n, k):
    """A CU cap under which the planner gives this shape 128x128 tiles with K split."""
    for cap in (8, 12, 16, 24, 32, 48, 64):
        plan = dg._dense_plan_for_tests(m, n, k, cap)
        if (plan["bm"], plan["bn"]) == (128, 128) and plan["splits"] > 1:
            return cap, plan
    pytest.fail(f"no CU cap gives a 128x128 split plan for M={m} N={n} K={k}")


@pytest.mark.parametrize("m,n,out,with_c", [(128, 1005, "bf16", False), (100, 520, "fp32", True)])
def test_128_column_split_tile_ue8m0(m, n, out, with_c):
    """The UE8M0 entry point on the 128x128 split tile (block-scaled MFMAs, partials
    reduced in split order) against the UE8M0 oracle."""
    k = 8192
    cap, plan = _cap_for_128_column_split(m, n, k)
    note(f"ue8m0 128x128 split M={m} N={n} K={k} cap={cap} {out} C={with_c}: {plan}")
    x = gen_dense(m, n, k, seed=9 * m + n, with_c=with_c, out_dtype=out, scale_fmt="ue8m0")
    ref = oracle.ref_dense_ue8m0(x["a"], x["sfa"], x["b"], x["sfb"], x.get("c"))
    try:
        dg.set_num_cus(cap)
        d = run_dense(x, ld_d=1024)
    finally:
        dg.set_num_cus(0)
    oracle.assert_close(as_f64(d), ref, f"ue8m0 128x128 split M={m} N={n}")


def test_wgrad_on_128_column_split_tile():
    """The in-place weight-gradient entry point (D += A B^T, FP32) on the 128x128 split tile."""
    m, n, k = 128, 520, 8192
    cap, plan = _cap_for_128_column_split(m, n, k)
    note(f"wgrad 128x128 split M={m} N={n} K={k} cap={cap}: {plan}")
    x = gen_dense(m, n, k, seed=1401, with_c=True, out_dtype="fp32")
    a, sfa, b, sfb = _dev_inputs(x)
    d = to_dev(x["c"].astype(np.float32))
    try:
        dg.set_num_cus(cap)
        ws = dg.alloc_workspace(m, n, k)
        assert ws is not None and ws.numel() == plan["ws_bytes"]
        dg.wgrad_fp8_gemm_nt((a, sfa), (b, sfb), d, workspace=ws)
        torch.cuda.synchronize()
    finally:
        dg.set_num_cus(0)
    oracle.assert_close(as_f64(d), oracle.ref_dense(x["a"], x["sfa"], x["b"], x["sfb"], x["c"]),
                        "wgrad 128x128 split")
