"""CPU tests of the input generators and of the acceptance check."""

import numpy as np
import pytest
import torch

from oracle import tolerance_report, TOL_REL, TOL_RMS
from workloads import (DENSE_SWEEP, gen_contiguous, gen_dense, gen_masked, quantize_per_block,
                       quantize_per_row_block, sf_aligned_size, workload, WORKLOAD_NAMES)


def _dec(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_row_block_quantization_rule():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 384), dtype=np.float32)
    x[2, 128:256] = 0
    q, s = quantize_per_row_block(x)
    assert s.shape == (5, 3) and s.dtype == np.float32
    amax = np.abs(x.reshape(5, 3, 128)).max(-1)
    want = (amax / np.float32(448)).astype(np.float32)
    want[2, 1] = 1.0
    assert np.array_equal(s, want)
    back = _dec(q).reshape(5, 3, 128) * s[..., None]
    # E4M3 RNE: relative error <= 2^-4 for normals, absolute <= 2^-10 * s in the subnormal range
    err = np.abs(back - x.reshape(5, 3, 128))
    assert (err <= np.maximum(np.abs(x.reshape(5, 3, 128)) * 2 ** -4, 2 ** -10 * s[..., None]) + 1e-30).all()
    # each block's largest element maps to +-448 exactly
    assert (np.abs(_dec(q)).reshape(5, 3, 128).max(-1)[s != 1] == 448).all()


def test_block_quantization_partial_rows():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((130, 256), dtype=np.float32)
    q, s = quantize_per_block(x)
    assert s.shape == (2, 2)
    assert s[1, 0] == np.float32(np.abs(x[128:, :128]).max() / np.float32(448))


def test_dense_layout():
    x = gen_dense(10, 20, 256, seed=0)
    assert x["a"].shape == (10, 256) and x["a"].dtype == np.uint8
    assert x["sfa"].shape == (2, sf_aligned_size(10)) and (x["sfa"][:, 10:] == 0).all()
    assert x["b"].shape == (20, 256) and x["sfb"].shape == (1, 2)
    assert x["c"] is None
    y = gen_dense(10, 20, 256, seed=0)
    assert np.array_equal(x["a"], y["a"]) and np.array_equal(x["b"], y["b"])
    z = gen_dense(4, 8, 128, seed=1, with_c=True)
    # BF16 outputs get a C that is exactly representable in BF16
    assert np.array_equal(torch.from_numpy(z["c"]).to(torch.bfloat16).float().numpy(), z["c"])


def test_contiguous_layout():
    x = gen_contiguous(3, 16, 128, seed=0, m_sizes=[1, 128, 129])
    assert x["m_total"] == 128 + 128 + 256
    mi = x["m_indices"]
    assert (mi[:1] == 0).all() and (mi[1:128] == -1).all()
    assert (mi[128:256] == 1).all()
    assert (mi[256:385] == 2).all() and (mi[385:] == -1).all()
    assert not x["a"][mi == -1].any()  # zero padding rows
    assert (x["sfa"][:, :x["m_total"]][:, mi == -1] == 1).all()


def test_masked_poison_layout():
    x = gen_masked(2, 8, 16, 128, seed=0, masked_m=[3, 8], poison=True)
    assert (x["a"][0, 3:] == 0x7F).all() and np.isnan(x["sfa"][0][:, 3:8]).all()
    assert not np.isnan(x["sfa"][1][:, :8]).any()


def test_dense_sweep_definition():
    assert len(DENSE_SWEEP) == 15
    assert DENSE_SWEEP[0] == (64, 2112, 7168) and DENSE_SWEEP[14] == (4096, 7168, 2048)
    for name in WORKLOAD_NAMES:
        assert len(workload(name)) >= 1


def test_tolerance_report_bounds():
    rng = np.random.default_rng(5)
    ref = rng.standard_normal(10000)
    rms = np.sqrt(np.mean(ref ** 2))
    ok = ref + 0.9 * (TOL_REL * np.abs(ref) + TOL_RMS * rms) * np.sign(rng.standard_normal(10000))
    rep = tolerance_report(ok, ref)
    assert rep["worst_ratio"] <= 1.0
    bad = ref.copy()
    bad[17] += 2 * (TOL_REL * abs(ref[17]) + TOL_RMS * rms)
    assert not tolerance_report(bad, ref)["ok"]
    nan = ref.copy()
    nan[3] = np.nan
    assert not tolerance_report(nan, ref)["ok"]
    assert tolerance_report(np.zeros(0), np.zeros(0))["ok"]
    # a tiny global scale error passes elementwise but is caught by cosine when large enough
    assert not tolerance_report(-ref, ref)["ok"]
