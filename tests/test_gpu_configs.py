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


# Output tile sizes the dispatcher can pick: 256-row tiles of 256, 224 or 160
# columns (the skinny and 128-row tiles divide these).
ROW_PERIODS = (256,)
COL_PERIODS = (256, 224, 160)


def _cover(rng, total, periods, valid=None, must=()):
    """Indices in [0, total) such that, for every period p, every residue mod p
    that occurs among the (valid) indices is present at least once, each taken
    from a randomly chosen tile; plus ``must``."""
    pick = set(int(v) for v in must if 0 <= v < total and (valid is None or valid[v]))
    for p in periods:
        idx = np.arange(total)
        for r in range(min(p, total)):
            cand = idx[r::p]
            if valid is not None:
                cand = cand[valid[cand]]
            if len(cand):
                pick.add(int(rng.choice(cand)))
    return np.array(sorted(pick))


def _assert_covers(idx, total, periods, valid=None, what=""):
    ok = np.ones(total, bool) if valid is None else valid
    for p in periods:
        need = set(np.nonzero(ok)[0] % p)
        got = set(np.asarray(idx) % p)
        assert need <= got, f"{what}: residues mod {p} not compared: {sorted(need - got)[:8]}"


@pytest.mark.parametrize("i", range(len(DENSE_SWEEP)))
def test_dense_sweep_full_size(i):
    m, n, k = DENSE_SWEEP[i]
    note(f"dense sweep case {i}: M={m} N={n} K={k} seed={100 + i}")
    x = gen_dense(m, n, k, seed=100 + i)
    d = run_dense(x)
    assert torch.isfinite(d.float()).all()
    rng = np.random.default_rng(1000 + i)
    rows = _cover(rng, m, ROW_PERIODS, must=(0, m - 1))
    cols = _cover(rng, n, COL_PERIODS, must=range(n - 70, n))
    _assert_covers(rows, m, ROW_PERIODS, what="rows")
    _assert_covers(cols, n, COL_PERIODS, what="cols")
    ref = oracle.ref_dense(x["a"], x["sfa"], x["b"], x["sfb"], rows=rows, cols=cols)
    rep = oracle.assert_close(take(d, rows, cols), ref, f"dense M={m} N={n} K={k}")
    note(f"  worst={rep['worst_ratio']:.3f} cos_dist={rep['cos_dist']:.2e} sampled={rep['n']}")


def test_dense_long_k_with_c_full_size():
    note("dense+C M=8192 N=8192 K=16384 FP32, seed=4")
    x = gen_dense(8192, 8192, 16384, seed=4, with_c=True, out_dtype="fp32")
    d = run_dense(x)
    assert torch.isfinite(d).all()
    rng = np.random.default_rng(44)
    rows = _cover(rng, 8192, ROW_PERIODS, must=(0, 8191))
    cols = _cover(rng, 8192, COL_PERIODS, must=(0, 8191))
    _assert_covers(rows, 8192, ROW_PERIODS, what="rows")
    _assert_covers(cols, 8192, COL_PERIODS, what="cols")
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
    rows = _cover(rng, x["m_total"], ROW_PERIODS, valid=written, must=np.concatenate([starts, ends, tail]))
    cols = _cover(rng, 4096, COL_PERIODS, must=(0, 4095))
    _assert_covers(rows, x["m_total"], ROW_PERIODS, valid=written, what="rows")
    _assert_covers(cols, 4096, COL_PERIODS, what="cols")
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
    groups = np.arange(16)  # every group, every valid row
    cols = _cover(rng, n, COL_PERIODS, must=(0, n - 1))
    _assert_covers(cols, n, COL_PERIODS, what="cols")
    ref, w = oracle.ref_masked(x["a"], x["sfa"], x["b"], x["sfb"], x["masked_m"], groups=groups, cols=cols)
    assert w.sum(axis=1).tolist() == [int(v) for v in mm], "every valid row of every group is compared"
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
    rows = _cover(rng, m, ROW_PERIODS, must=(0, m - 1))
    cols = _cover(rng, n, COL_PERIODS, must=range(n - 70, n))
    _assert_covers(rows, m, ROW_PERIODS, what="rows")
    _assert_covers(cols, n, COL_PERIODS, what="cols")
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
    rows = _cover(rng, x["m_total"], ROW_PERIODS, valid=written)
    cols = _cover(rng, 4096, COL_PERIODS, must=(0, 4095))
    _assert_covers(rows, x["m_total"], ROW_PERIODS, valid=written, what="rows")
    _assert_covers(cols, 4096, COL_PERIODS, what="cols")
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
    groups = np.arange(16)
    cols = _cover(rng, 4096, COL_PERIODS, must=(0, 4095))
    _assert_covers(cols, 4096, COL_PERIODS, what="cols")
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
    rows = _cover(rng, 4096, ROW_PERIODS, must=(0, 4095))
    cols = _cover(rng, 7168, COL_PERIODS, must=(0, 7167))
    _assert_covers(rows, 4096, ROW_PERIODS, what="rows")
    _assert_covers(cols, 7168, COL_PERIODS, what="cols")
    ref = oracle.ref_k_grouped(x["a"], x["sfa"], x["b"], x["sfb"], x["ks"], c=x["c"], rows=rows, cols=cols)
    for g in range(8):
        rep = oracle.assert_close(take(d[g], rows, cols), ref[g], f"k-grouped group {g}")
        note(f"  group {g} K={x['ks'][g]}: worst={rep['worst_ratio']:.3f} cos_dist={rep['cos_dist']:.2e}")
