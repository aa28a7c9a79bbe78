"""GPU parity of the scale-layout transform (dg_transform_sf_into_required_layout)
against the oracle's plain transform: a byte-for-byte copy, so the bar is bit
equality; columns past the rows keep their sentinel; the transformed scales
feed the GEMM and give the bits of the generator's own layout."""

import numpy as np
import pytest
import torch

import oracle
from workloads import gen_dense

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():  # pragma: no cover - GPU only
    from tests._gpu_harness import fp8_dev, note, raw_bits, run_dense, to_dev
    import moe_grouped_gemm_tiles_amd as dg


@pytest.mark.parametrize("g,mn,kb", [(1, 1, 1), (1, 70, 33), (3, 130, 5), (2, 64, 32), (1, 257, 130)])
@pytest.mark.parametrize("ue8m0", [False, True])
def test_transform_matches_oracle(g, mn, kb, ue8m0):
    note(f"layout g={g} mn={mn} kb={kb} ue8m0={ue8m0}")
    rng = np.random.default_rng(1000 + mn + kb)
    if ue8m0:
        sf = np.exp2(rng.integers(-30, 20, (g, mn, kb))).astype(np.float32)
    else:
        sf = rng.standard_normal((g, mn, kb)).astype(np.float32)
    got = dg.transform_sf_into_required_layout(to_dev(sf), ue8m0=ue8m0).cpu().numpy()
    ld = got.shape[-1]
    assert ld == (mn + 3) // 4 * 4
    want = oracle.transform_sf(sf, ld, ue8m0)
    assert np.array_equal(got[..., :mn].view(np.uint32), want[..., :mn].view(np.uint32))


def test_padding_columns_untouched():
    lib = dg.load_library()
    sf = to_dev(np.ones((6, 3), np.float32))
    out = torch.full((3, 12), float("nan"), device="cuda")
    assert lib.dg_transform_sf_into_required_layout(sf.data_ptr(), out.data_ptr(), 1, 6, 3, 12, 0, None) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert (o[:, :6] == 1.0).all() and np.isnan(o[:, 6:]).all()


def test_transformed_scales_drive_the_gemm():
    x = gen_dense(200, 384, 640, seed=97)
    want = raw_bits(run_dense(x))
    rows_sf = np.ascontiguousarray(x["sfa"][:, :200].T)  # back to per-row [m, kb]
    sfa = dg.transform_sf_into_required_layout(to_dev(rows_sf))
    d = torch.empty(200, 384, dtype=torch.bfloat16, device="cuda")
    dg.fp8_gemm_nt((fp8_dev(x["a"]), sfa), (fp8_dev(x["b"]), to_dev(x["sfb"])), d)
    torch.cuda.synchronize()
    assert np.array_equal(raw_bits(d), want)
