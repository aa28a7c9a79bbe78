"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.  The oracle evaluates sampled rows x columns (it computes
each sampled output from its own row and column only); whole-output
properties (no NaN/Inf in written rows, unwritten rows keep the sentinel)
are checked everywhere.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import DENSE_SWEEP, gen_contiguous, gen_dense, gen_k_grouped, gen_masked

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():  # pragma: no cover - GPU only
    from tests._gpu_harness import (as_f64, note, raw_bits, run_contiguous, run_dense, run_k_grouped, run_masked,
                                    sentinel_of, take)


def _sample(rng, total, count, must=()):
    pick = set(int(v) for v in must if 0 <= v < total)
    if total <= count:
        return np.arange(total)
    pick.update(rng.choice(total, count, replace=False).tolist())
    return np.array(sorted(pick))


@pytest.mark.parametrize("i", range(len(DENSE_SWEEP)))
def test_dense_sweep_full_size(i):
    m, n, k = DENSE_SWEEP[i]
    note(f"dense sweep case {i}: M={m} N={n} K={k} seed={100 + i}")
    x = gen_dense(m, n, k, seed=100 + i)
    d = run_dense(x)
    assert torch.isfinite(d.float()).all()
    rng = np.random.default_rng(1000 + i)
    rows = _sample(rng, m, 48, must=(0, m - 1))
    cols = _sample(rng, n, 768, must=range(n - 70, n))
    ref = oracle.ref_dense(x["a"], x["sfa"], x["b"], x["sfb"], rows=rows, cols=cols)
    rep = oracle.assert_close(take(d, rows, cols), ref, f"dense M={m} N={n} K={k}")
    note(f"  worst={rep['worst_ratio']:.3f} cos_dist={rep['cos_dist']:.2e} sampled={rep['n']}")


def test_dense_long_k_with_c_full_size():
    note("dense+C M=8192 N=8192 K=16384 FP32, seed=4")
    x = gen_dense(8192, 8192, 16384, seed=4, with_c=True, out_dtype="fp32")
    d = run_dense(x)
    assert torch.isfinite(d).all()
    rng = np.random.default_rng(44)
    rows = _sample(rng, 8192, 24, must=(0, 8191))
    cols = _sample(rng, 8192, 512, must=(0, 8191))
    ref = oracle.ref_dense(x["a"], x["sfa"], x["b"], x["sfb"], x["c"], rows=rows, cols=cols)
    rep = oracle.assert_close(take(d, rows, cols), ref, "dense+C long K")
    note(f"  worst={rep['worst_ratio']:.3f} cos_dist={rep['cos_dist']:.2e}")


def test_contiguous_moe_full_size():
    note("contiguous G=8 N=4096 K=7168, seed=2")
    x = gen_contiguous(8, 4096, 7168, seed=2)
    d = run_contiguous(x)
    mi = x["m_indices"]
    written = mi >= 0
    bits = raw_bits(d)
    assert (bits[~written] == sentinel_of(d)).all()
    assert torch.isfinite(d[torch.from_numpy(written).to(d.device)].float()).all()
    rng = np.random.default_rng(22)
    starts = np.concatenate([[0], np.cumsum([-(-int(s) // 128) * 128 for s in x["m_sizes"]])[:-1]])
    ends = starts + x["m_sizes"] - 1
    # rows of the last 512, which a ragged last round sends to the 128x128 launch
    tail = x["m_total"] - np.array([512, 511, 384, 257, 256, 129, 1])
    rows = _sample(rng, x["m_total"], 64, must=np.concatenate([starts, ends, tail]))
    rows = rows[written[rows]]
    cols = _sample(rng, 4096, 512, must=(0, 4095))
    ref, w = oracle.ref_contiguous(x["a"], x["sfa"], x["b"], x["sfb"], mi, rows=rows, cols=cols)
    assert w.all()
    rep = oracle.assert_close(take(d, rows, cols), ref, "contiguous full size")
    note(f"  worst={rep['worst_ratio']:.3f} cos_dist={rep['cos_dist']:.2e} rows_total={written.sum()}")


@pytest.mark.parametrize("j,n,k", [(0, 4096, 7168), (1, 7168, 2048)])
@pytest.mark.parametrize("poison", [False, True])
def test_masked_decode_full_size(j, n, k, poison):
    note(f"masked G=16 Mmax=256 N={n} K={k} seed={30 + j} poison={poison}")
    x = gen_masked(16, 256, n, k, seed=30 + j, poison=poison)
    d = run_masked(x, expected_m=128)
    mm = np.clip(x["masked_m"], 0, 256)
    written = np.arange(256)[None, :] < mm[:, None]
    bits = raw_bits(d)
    assert (bits[~written] == sentinel_of(d)).all()
    assert torch.isfinite(d[torch.from_numpy(written).to(d.device)].float()).all()
    rng = np.random.default_rng(300 + j)
    groups = rng.choice(16, 4, replace=False)
    cols = _sample(rng, n, 512, must=(0, n - 1))
    ref, w = oracle.ref_masked(x["a"], x["sfa"], x["b"], x["sfb"], x["masked_m"], groups=groups, cols=cols)
    got = np.stack([take(d[int(g)], np.arange(256), cols) for g in groups])
    rep = oracle.assert_close(got[w], ref[w], f"masked full size j={j}")
    note(f"  worst={rep['worst_ratio']:.3f} cos_dist={rep['cos_dist']:.2e} masked_m={x['masked_m'].tolist()}")


@pytest.mark.parametrize("i", [2, 7, 11, 12])
def test_dense_sweep_ue8m0_full_size(i):
    m, n, k = DENSE_SWEEP[i]
    note(f"dense ue8m0 sweep case {i}: M={m} N={n} K={k} seed={100 + i}")
    x = gen_dense(m, n, k, seed=100 + i, scale_fmt="ue8m0")
    d = run_dense(x)
    assert torch.isfinite(d.float()).all()
    rng = np.random.default_rng(2000 + i)
    rows = _sample(rng, m, 48, must=(0, m - 1))
    cols = _sample(rng, n, 768, must=range(n - 70, n))
    ref = oracle.ref_dense_ue8m0(x["a"], x["sfa"], x["b"], x["sfb"], rows=rows, cols=cols)
    rep = oracle.assert_close(take(d, rows, cols), ref, f"dense ue8m0 M={m} N={n} K={k}")
    note(f"  worst={rep['worst_ratio']:.3f} cos_dist={rep['cos_dist']:.2e} sampled={rep['n']}")


def test_contiguous_moe_ue8m0_full_size():
    note("contiguous ue8m0 G=8 N=4096 K=7168, seed=2")
    x = gen_contiguous(8, 4096, 7168, seed=2, scale_fmt="ue8m0")
    d = run_contiguous(x)
    mi = x["m_indices"]
    written = mi >= 0
    assert (raw_bits(d)[~written] == sentinel_of(d)).all()
    rng = np.random.default_rng(23)
    rows = _sample(rng, x["m_total"], 64, must=())
    rows = rows[written[rows]]
    cols = _sample(rng, 4096, 512, must=(0, 4095))
    ref, w = oracle.ref_contiguous_ue8m0(x["a"], x["sfa"], x["b"], x["sfb"], mi, rows=rows, cols=cols)
    assert w.all()
    rep = oracle.assert_close(take(d, rows, cols), ref, "contiguous ue8m0 full size")
    note(f"  worst={rep['worst_ratio']:.3f} cos_dist={rep['cos_dist']:.2e}")


def test_masked_decode_ue8m0_full_size():
    note("masked ue8m0 G=16 Mmax=256 N=4096 K=7168 seed=30")
    x = gen_masked(16, 256, 4096, 7168, seed=30, scale_fmt="ue8m0")
    d = run_masked(x, expected_m=128)
    mm = np.clip(x["masked_m"], 0, 256)
    written = np.arange(256)[None, :] < mm[:, None]
    assert (raw_bits(d)[~written] == sentinel_of(d)).all()
    rng = np.random.default_rng(301)
    groups = rng.choice(16, 3, replace=False)
    cols = _sample(rng, 4096, 512, must=(0, 4095))
    ref, w = oracle.ref_masked_ue8m0(x["a"], x["sfa"], x["b"], x["sfb"], x["masked_m"], groups=groups, cols=cols)
    got = np.stack([take(d[int(g)], np.arange(256), cols) for g in groups])
    rep = oracle.assert_close(got[w], ref[w], "masked ue8m0 full size")
    note(f"  worst={rep['worst_ratio']:.3f} cos_dist={rep['cos_dist']:.2e}")


def test_k_grouped_wgrad_full_size():
    note("k-grouped G=8 M=4096 N=7168 K_g~U[1,8192] seed=5, D = C + A_g B_g^T")
    x = gen_k_grouped(8, 4096, 7168, seed=5)
    note(f"  ks={x['ks'].tolist()} K_total={x['k']}")
    d = run_k_grouped(x, with_c=True)
    assert torch.isfinite(d).all()
    rng = np.random.default_rng(55)
    rows = _sample(rng, 4096, 24, must=(0, 4095))
    cols = _sample(rng, 7168, 384, must=(0, 7167))
    ref = oracle.ref_k_grouped(x["a"], x["sfa"], x["b"], x["sfb"], x["ks"], c=x["c"], rows=rows, cols=cols)
    for g in range(8):
        rep = oracle.assert_close(take(d[g], rows, cols), ref[g], f"k-grouped group {g}")
        note(f"  group {g} K={x['ks'][g]}: worst={rep['worst_ratio']:.3f} cos_dist={rep['cos_dist']:.2e}")
