"""Pins for the FP64 GEMM oracle (CPU only).

Each pin checks the oracle against something other than itself:

* exact brute force in rationals (``fractions.Fraction``) on tiny shapes for
  all three variants, decoding bytes with torch's independent E4M3 decoder;
* unit scales reduce the oracle to a plain library matmul of decoded bytes;
* one-hot A rows select single B entries exactly (also with power-of-two
  scales);
* slab additivity and single-slab isolation (sum over 128-K slabs, and a
  slab's result ignores the other slabs' bytes);
* scale linearity (doubling one row scale / one block scale doubles exactly
  that row / that 128-column block);
* zero A gives exactly C;
* grouped = per-group dense, with unwritten rows reported;
* planted mistakes in the oracle (wrong exponent bias, transposed scale
  index, dropped C, off-by-one mask) are caught by these pins.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import oracle.gemm as og
from oracle import ref_dense, ref_contiguous, ref_masked
from workloads import gen_dense, gen_contiguous, gen_masked, sf_to_mn_major


# ----------------------------------------------------------------- helpers

def _exact_vals(codes: np.ndarray):
    """Exact rationals of E4M3 codes via torch's decoder (independent of the oracle table)."""
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64)
    return np.vectorize(Fraction, otypes=[object])(t.numpy())


def _brute_dense(a, sfa, b, sfb, c=None, rows=None):
    """Exact D by triple loop; returns (exact values, sum of |terms|) as float arrays."""
    m_all, k = a.shape
    n = b.shape[0]
    rows = range(m_all) if rows is None else rows
    va, vb = _exact_vals(a), _exact_vals(b)
    out = np.zeros((len(rows), n))
    mag = np.zeros((len(rows), n))
    for i, m in enumerate(rows):
        for j in range(n):
            s = Fraction(0)
            s_abs = Fraction(0)
            for kk in range(k):
                t = (va[m, kk] * Fraction(float(sfa[kk // 128, m]))
                     * vb[j, kk] * Fraction(float(sfb[j // 128, kk // 128])))
                s += t
                s_abs += abs(t)
            if c is not None:
                s += Fraction(float(c[m, j]))
                s_abs += abs(Fraction(float(c[m, j])))
            out[i, j] = float(s)
            mag[i, j] = float(s_abs)
    return out, mag


def _close_to_exact(got, exact, mag, rel=1e-12):
    return bool(np.all(np.abs(got - exact) <= rel * mag + 1e-300))


def _pin_dense_bruteforce(seed=7, m=5, n=6, k=384, with_c=True):
    x = gen_dense(m, n, k, seed=seed, with_c=with_c, out_dtype="fp32")
    exact, mag = _brute_dense(x["a"], x["sfa"], x["b"], x["sfb"], x["c"])
    got = ref_dense(x["a"], x["sfa"], x["b"], x["sfb"], x["c"])
    return _close_to_exact(got, exact, mag)


# ------------------------------------------------------------ brute force

@pytest.mark.parametrize("m,n,k,with_c", [(5, 6, 128, False), (8, 8, 256, True), (3, 7, 384, True)])
def test_dense_matches_exact_bruteforce(m, n, k, with_c):
    x = gen_dense(m, n, k, seed=11 + m, with_c=with_c, out_dtype="fp32")
    exact, mag = _brute_dense(x["a"], x["sfa"], x["b"], x["sfb"], x["c"])
    got = ref_dense(x["a"], x["sfa"], x["b"], x["sfb"], x["c"])
    assert _close_to_exact(got, exact, mag)


def test_dense_partial_column_block_bruteforce():
    # N = 130 -> the second 128-row block of B holds 2 rows and has its own scale
    x = gen_dense(2, 130, 256, seed=5)
    exact, mag = _brute_dense(x["a"], x["sfa"], x["b"], x["sfb"])
    got = ref_dense(x["a"], x["sfa"], x["b"], x["sfb"])
    assert x["sfb"].shape == (2, 2)
    assert _close_to_exact(got, exact, mag)


def test_dense_padded_sfa_leading_dim():
    # ld_sfa larger than M: padding columns must be ignored
    x = gen_dense(3, 4, 256, seed=9, ld_sfa=12)
    x["sfa"][:, 3:] = np.nan
    exact, mag = _brute_dense(x["a"], x["sfa"], x["b"], x["sfb"])
    got = ref_dense(x["a"], x["sfa"], x["b"], x["sfb"])
    assert _close_to_exact(got, exact, mag)


def test_contiguous_matches_exact_bruteforce():
    x = gen_contiguous(3, 6, 256, seed=21, m_sizes=[3, 0, 5])
    assert x["m_total"] == 256
    ref, written = ref_contiguous(x["a"], x["sfa"], x["b"], x["sfb"], x["m_indices"])
    mi = x["m_indices"]
    assert written.sum() == 8
    assert (written == (mi >= 0)).all()
    for g in range(3):
        rows = [r for r in range(x["m_total"]) if mi[r] == g]
        if not rows:
            continue
        exact, mag = _brute_dense(x["a"], x["sfa"], x["b"][g], x["sfb"][g], rows=rows)
        assert _close_to_exact(ref[rows], exact, mag)
    assert np.isnan(ref[~written]).all()


def test_masked_matches_exact_bruteforce():
    x = gen_masked(4, 6, 5, 128, seed=31, masked_m=[0, 9, 3, -2])
    ref, written = ref_masked(x["a"], x["sfa"], x["b"], x["sfb"], x["masked_m"])
    assert written.sum(axis=1).tolist() == [0, 6, 3, 0]  # clamped to [0, M_max]
    for g in range(4):
        mm = int(written[g].sum())
        if mm == 0:
            continue
        exact, mag = _brute_dense(x["a"][g], x["sfa"][g], x["b"][g], x["sfb"][g], rows=list(range(mm)))
        assert _close_to_exact(ref[g, :mm], exact, mag)
    assert np.isnan(ref[~written]).all()


# ------------------------------------------------------------- unit scales

def test_unit_scales_reduce_to_library_matmul():
    rng = np.random.default_rng(3)
    m, n, k = 33, 70, 256
    a = rng.integers(0, 256, (m, k), dtype=np.uint8)
    b = rng.integers(0, 256, (n, k), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0  # no NaN codes
    b[(b & 0x7F) == 0x7F] = 0
    sfa = np.ones((k // 128, 36), np.float32)
    sfb = np.ones((1, k // 128), np.float32)
    at = torch.from_numpy(a).view(torch.float8_e4m3fn).to(torch.float64)
    bt = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64)
    want = (at @ bt.T).numpy()
    got = ref_dense(a, sfa, b, sfb)
    assert np.allclose(got, want, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- one-hot

@pytest.mark.parametrize("pow2", [False, True])
def test_one_hot_selects_single_entries(pow2):
    rng = np.random.default_rng(4)
    m, n, k = 20, 150, 384
    perm = rng.permutation(k)[:m]
    a = np.zeros((m, k), np.uint8)
    a[np.arange(m), perm] = 0x38  # 1.0
    b = rng.integers(0, 256, (n, k), dtype=np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x38
    kb, nb = k // 128, 2
    if pow2:
        ea = rng.integers(-4, 5, (kb, m))
        eb = rng.integers(-4, 5, (nb, kb))
        sfa = np.ldexp(np.ones((kb, m)), ea).astype(np.float32)
        sfb = np.ldexp(np.ones((nb, kb)), eb).astype(np.float32)
    else:
        ea = np.zeros((kb, m), int)
        eb = np.zeros((nb, kb), int)
        sfa = np.ones((kb, m), np.float32)
        sfb = np.ones((nb, kb), np.float32)
    sfa_p = np.zeros((kb, 20), np.float32)
    sfa_p[:, :m] = sfa
    got = ref_dense(a, sfa_p, b, sfb)
    bt = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for i in range(m):
        kk = perm[i]
        for j in range(n):
            want = np.ldexp(bt[j, kk], int(ea[kk // 128, i] + eb[j // 128, kk // 128]))
            assert got[i, j] == want


# ------------------------------------------------- slabs and scale linearity

def test_slab_additivity_and_isolation():
    x = gen_dense(9, 140, 512, seed=13)
    a, sfa, b, sfb = x["a"], x["sfa"], x["b"], x["sfb"]
    total = ref_dense(a, sfa, b, sfb)
    parts = []
    for j in range(4):
        s = sfa.copy()
        s[np.arange(4) != j] = 0.0
        dj = ref_dense(a, s, b, sfb)
        # bytes of other slabs must not matter once their scale is zero
        a2, b2 = a.copy(), b.copy()
        other = np.ones(512, bool)
        other[j * 128:(j + 1) * 128] = False
        a2[:, other] = 0x38
        b2[:, other] = 0x40
        assert np.array_equal(ref_dense(a2, s, b2, sfb), dj)
        parts.append(dj)
    assert np.allclose(sum(parts), total, rtol=1e-12, atol=1e-12 * np.abs(total).max())


def test_scale_linearity():
    x = gen_dense(6, 300, 256, seed=17)
    a, sfa, b, sfb = x["a"], x["sfa"], x["b"], x["sfb"]
    base = ref_dense(a, sfa, b, sfb)
    s = sfa.copy()
    s[:, 4] *= 2
    d = ref_dense(a, s, b, sfb)
    assert np.array_equal(d[4], 2 * base[4])
    assert np.array_equal(np.delete(d, 4, 0), np.delete(base, 4, 0))
    t = sfb.copy()
    t[1, :] *= 2  # columns 128..255
    d = ref_dense(a, sfa, b, t)
    assert np.array_equal(d[:, 128:256], 2 * base[:, 128:256])
    assert np.array_equal(d[:, :128], base[:, :128]) and np.array_equal(d[:, 256:], base[:, 256:])


def test_zero_a_gives_c():
    x = gen_dense(7, 50, 256, seed=19, with_c=True, out_dtype="fp32")
    a0 = np.zeros_like(x["a"])
    assert np.array_equal(ref_dense(a0, x["sfa"], x["b"], x["sfb"], x["c"]), x["c"].astype(np.float64))
    assert not ref_dense(a0, x["sfa"], x["b"], x["sfb"]).any()


# ------------------------------------------------------ grouped = dense

def test_contiguous_equals_per_group_dense():
    x = gen_contiguous(4, 200, 256, seed=23, m_sizes=[130, 1, 0, 127])
    ref, written = ref_contiguous(x["a"], x["sfa"], x["b"], x["sfb"], x["m_indices"])
    off = 0
    for g, s in enumerate(x["m_sizes"]):
        s = int(s)
        rows = np.arange(off, off + s)
        a_g = x["a"][rows]
        sfa_g = sf_to_mn_major(x["sfa"][:, rows].T)
        want = ref_dense(a_g, sfa_g, x["b"][g], x["sfb"][g])
        assert np.array_equal(ref[rows], want)
        off += -(-s // 128) * 128
    assert written.sum() == 258


def test_masked_equals_per_group_dense():
    x = gen_masked(3, 40, 130, 256, seed=29, masked_m=[40, 17, 0], poison=True)
    ref, written = ref_masked(x["a"], x["sfa"], x["b"], x["sfb"], x["masked_m"])
    for g, mm in enumerate([40, 17, 0]):
        if mm:
            sfa_g = sf_to_mn_major(x["sfa"][g][:, :mm].T)
            want = ref_dense(x["a"][g][:mm], sfa_g, x["b"][g], x["sfb"][g])
            assert np.array_equal(ref[g, :mm], want)
            assert np.isfinite(ref[g, :mm]).all()  # poison rows do not leak
        assert not written[g, mm:].any()


# ---------------------------------------------------- planted mistakes

def test_planted_wrong_exponent_bias_is_caught(monkeypatch):
    bad = np.array([oracle.e4m3_closed_form(c) * (0.5 if (c & 0x78) else 1.0) for c in range(256)])
    monkeypatch.setattr(og, "decode_e4m3", lambda codes: bad[codes])
    assert not _pin_dense_bruteforce()


def test_planted_transposed_block_scale_is_caught(monkeypatch):
    real = og.dequant_b

    def swapped(b, sfb, cols=None):
        return real(b, np.ascontiguousarray(sfb.T) if sfb.shape[0] == sfb.shape[1] else sfb[::-1], cols)

    monkeypatch.setattr(og, "dequant_b", swapped)
    # N = 256, K = 256 -> sfb is 2x2 and a transposed index still runs
    x = gen_dense(2, 256, 256, seed=41)
    exact, mag = _brute_dense(x["a"], x["sfa"], x["b"], x["sfb"])
    got = og.ref_dense(x["a"], x["sfa"], x["b"], x["sfb"])
    assert not _close_to_exact(got, exact, mag)


def test_planted_dropped_c_is_caught(monkeypatch):
    real = og.ref_dense
    monkeypatch.setattr(og, "ref_dense", lambda a, sfa, b, sfb, c=None, rows=None, cols=None:
                        real(a, sfa, b, sfb, None, rows, cols))
    x = gen_dense(7, 50, 256, seed=19, with_c=True, out_dtype="fp32")
    a0 = np.zeros_like(x["a"])
    assert not np.array_equal(og.ref_dense(a0, x["sfa"], x["b"], x["sfb"], x["c"]), x["c"].astype(np.float64))


def test_planted_mask_off_by_one_is_caught(monkeypatch):
    x = gen_masked(2, 6, 4, 128, seed=43, masked_m=[3, 6])
    real = og.ref_dense

    def shifted(a, sfa, b, sfb, c=None, rows=None, cols=None):
        if rows is not None:
            rows = np.minimum(np.asarray(rows) + 1, a.shape[0] - 1)
        return real(a, sfa, b, sfb, c, rows, cols)

    monkeypatch.setattr(og, "ref_dense", shifted)
    ref, _ = og.ref_masked(x["a"], x["sfa"], x["b"], x["sfb"], x["masked_m"])
    exact, mag = _brute_dense(x["a"][0], x["sfa"][0], x["b"][0], x["sfb"][0], rows=[0, 1, 2])
    assert not _close_to_exact(ref[0, :3], exact, mag)
