"""Pins of the oracle's scale-layout transform (oracle/layout.py), CPU only.

The transform is pinned through what the layouts mean rather than by
re-typing it: a GEMM whose A scales come out of the transform must equal the
GEMM written with the per-row scales applied element by element; the packed
UE8M0 form, decoded by the independent UE8M0 oracle, must give the same GEMM
as the FP32 form of the same powers of two; and the exponent bytes of a few
powers of two are fixed by the FP32 format.
"""

import numpy as np

import oracle
from oracle.e4m3 import decode_e4m3
from oracle.layout import transform_sf
from workloads import pack_ue8m0


def _codes(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3A  # no NaN codes
    return c


def test_fp32_layout_means_row_scales():
    rng = np.random.default_rng(1)
    m, n, k = 13, 9, 384
    kb = k // 128
    a, b = _codes(rng, (m, k)), _codes(rng, (n, k))
    sf_rows = rng.uniform(0.01, 4.0, (m, kb)).astype(np.float32)
    sfb = rng.uniform(0.01, 4.0, (1, kb)).astype(np.float32)
    # definition: A's element (m, k) is dec(A[m, k]) * sf_rows[m, k // 128]
    ad = decode_e4m3(a) * np.repeat(sf_rows.astype(np.float64), 128, axis=1)
    bd = decode_e4m3(b) * np.repeat(sfb.astype(np.float64), 128, axis=1)[0]
    want = ad @ bd.T
    for ld in (16, 20):
        got = oracle.ref_dense(a, transform_sf(sf_rows, ld), b, sfb)
        assert np.allclose(got, want, rtol=1e-13, atol=0)


def test_fp32_layout_grouped_is_per_group():
    rng = np.random.default_rng(2)
    sf = rng.uniform(0.1, 2.0, (3, 5, 7)).astype(np.float32)
    out = transform_sf(sf, 8)
    assert out.shape == (3, 7, 8)
    for g in range(3):
        one = transform_sf(sf[g], 8)
        assert np.array_equal(out[g][:, :5], one[:, :5])


def test_ue8m0_packing_matches_fp32_form():
    rng = np.random.default_rng(3)
    m, n, k = 11, 6, 640  # 5 K blocks: the last word holds one block and three padding bytes
    kb = k // 128
    a, b = _codes(rng, (m, k)), _codes(rng, (n, k))
    sf_rows = np.exp2(rng.integers(-12, 6, (m, kb))).astype(np.float32)
    sfb = np.exp2(rng.integers(-6, 3, (1, kb))).astype(np.float32)
    ld = 12
    fp32 = oracle.ref_dense(a, transform_sf(sf_rows, ld), b, sfb)
    ue = oracle.ref_dense_ue8m0(a, transform_sf(sf_rows, ld, ue8m0=True), b, pack_ue8m0(sfb, axis=1))
    assert np.array_equal(fp32, ue)


def test_ue8m0_bytes_of_powers_of_two():
    sf = np.array([[2.0 ** -3, 1.0, 2.0 ** 5, 0.5, 2.0 ** -20]], dtype=np.float32)
    w = transform_sf(sf, 4, ue8m0=True).view(np.uint32)
    assert w.shape == (2, 4)
    assert [(int(w[0, 0]) >> (8 * j)) & 0xFF for j in range(4)] == [124, 127, 132, 126]
    assert [(int(w[1, 0]) >> (8 * j)) & 0xFF for j in range(4)] == [107, 127, 127, 127]  # padding bytes 127


def test_planted_transposition_is_caught():
    rng = np.random.default_rng(4)
    m, n, k = 8, 4, 512
    kb = k // 128
    a, b = _codes(rng, (m, k)), _codes(rng, (n, k))
    sf_rows = rng.uniform(0.1, 3.0, (m, kb)).astype(np.float32)
    sfb = np.ones((1, kb), np.float32)
    good = oracle.ref_dense(a, transform_sf(sf_rows, 8), b, sfb)
    # the mistake a transform could make: K blocks and rows swapped in the output
    bad_sfa = np.zeros((kb, 8), np.float32)
    bad_sfa[:, :m] = sf_rows.reshape(kb, m)
    bad = oracle.ref_dense(a, bad_sfa, b, sfb)
    assert not np.allclose(good, bad)
