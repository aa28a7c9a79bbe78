"""Pins for the oracle's UE8M0, K-grouped, quantization and MQA-logits parts (CPU only).

Each pin checks the oracle against something other than itself:

* UE8M0 decode against torch's independent ``float8_e8m0fnu`` decoder on all
  256 bytes; word unpacking against a little-endian byte view of the words;
  the UE8M0 GEMM against exact rational brute force and against the FP32-scale
  GEMM with the same powers of two;
* K-grouped GEMM: group results add up to the dense GEMM over all of K,
  one group equals the dense GEMM, empty groups give exactly C, and a tiny
  case matches exact rational brute force;
* quantization: the E4M3 rounding agrees code-for-code with torch's cast on
  every code value, every midpoint and the FP32 neighbours of each midpoint;
  whole tensors agree with an independent torch-based quantizer; the scale
  rule, error bound and layouts are checked as properties;
* MQA logits: exact rational brute force on tiny inputs (with empty and
  clamped ranges), ReLU placement (negating kv), linearity in the weights,
  and the -inf / untouched marking outside the ranges;
* planted mistakes in the oracle are caught by these pins.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import oracle.kgrouped as okg
import oracle.mqa as omqa
import oracle.quant as oq
import oracle.ue8m0 as oue
from workloads import quantize_per_block, quantize_per_row_block, sf_to_mn_major


def _exact_e4m3(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64)
    return np.vectorize(Fraction, otypes=[object])(t.numpy())


# --------------------------------------------------------------------- UE8M0

def test_ue8m0_table_matches_torch_on_all_bytes():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    tab = oue.UE8M0_TABLE
    assert np.isnan(tab[255]) and np.isnan(t[255])
    assert np.array_equal(tab[:255], t[:255])
    assert tab[127] == 1.0 and tab[0] == 2.0 ** -127 and tab[254] == 2.0 ** 127


def test_unpack_matches_little_endian_byte_view():
    rng = np.random.default_rng(0)
    words = rng.integers(0, 2 ** 32, (3, 5), dtype=np.uint64).astype(np.uint32).view(np.int32)
    # along the last axis: bytes in memory order are the blocks in K order
    got = oue.unpack_ue8m0(words, kb=18, axis=1)
    want = np.ascontiguousarray(words).view(np.uint8).reshape(3, 20)[:, :18]
    assert np.array_equal(got, want)
    # along the first axis (MN-major A scales): word [q][m], byte j -> block 4q + j
    got0 = oue.unpack_ue8m0(words, kb=10, axis=0)
    want0 = np.ascontiguousarray(words.T).view(np.uint8).reshape(5, 12)[:, :10].T
    assert np.array_equal(got0, want0)


def _pack_test_side(e, axis):
    """Independent packer for the tests: little-endian byte view, padding 127."""
    e = np.moveaxis(np.asarray(e, np.uint8), axis, -1)
    kb = e.shape[-1]
    kq = (kb + 3) // 4
    buf = np.full((*e.shape[:-1], 4 * kq), 127, np.uint8)
    buf[..., :kb] = e
    w = np.ascontiguousarray(buf).view(np.int32)
    return np.moveaxis(w, -1, axis)


def test_ue8m0_gemm_brute_force_and_fp32_equivalence():
    rng = np.random.default_rng(1)
    m, n, k = 5, 130, 384
    a = rng.integers(0, 256, (m, k), dtype=np.uint8)
    b = rng.integers(0, 256, (n, k), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x30
    b[(b & 0x7F) == 0x7F] = 0x31
    kb, nb = k // 128, 2
    ea = rng.integers(120, 135, (kb, m)).astype(np.uint8)
    eb = rng.integers(120, 135, (nb, kb)).astype(np.uint8)
    sfa_w = _pack_test_side(ea, axis=0)
    sfb_w = _pack_test_side(eb, axis=1)
    got = oue.ref_dense_ue8m0(a, sfa_w, b, sfb_w)
    # equals the FP32-scale oracle with the same powers of two
    sfa_f = np.ldexp(np.float32(1), ea.astype(np.int32) - 127).astype(np.float32)
    sfb_f = np.ldexp(np.float32(1), eb.astype(np.int32) - 127).astype(np.float32)
    assert np.array_equal(got, oracle.ref_dense(a, sfa_f, b, sfb_f))
    # exact brute force on a few entries
    va, vb = _exact_e4m3(a), _exact_e4m3(b)
    for i, j in [(0, 0), (4, 129), (2, 77)]:
        s = sum(va[i, kk] * vb[j, kk] * Fraction(2) ** (int(ea[kk // 128, i]) + int(eb[j // 128, kk // 128]) - 254)
                for kk in range(k))
        assert got[i, j] == pytest.approx(float(s), rel=1e-12, abs=1e-300)


def test_ue8m0_grouped_variants_equal_fp32_variants():
    rng = np.random.default_rng(2)
    g, mm, n, k = 3, 64, 256, 640
    kb, kq = k // 128, (k // 128 + 3) // 4
    a = rng.integers(0, 0x7E, (g, mm, k), dtype=np.uint8)
    b = rng.integers(0, 0x7E, (g, n, k), dtype=np.uint8)
    ea = rng.integers(110, 140, (g, kb, mm)).astype(np.uint8)
    eb = rng.integers(110, 140, (g, n // 128, kb)).astype(np.uint8)
    fa = np.ldexp(1.0, ea.astype(int) - 127)
    fb = np.ldexp(1.0, eb.astype(int) - 127)
    wa = _pack_test_side(ea, axis=1)
    wb = _pack_test_side(eb, axis=2)
    assert wa.shape == (g, kq, mm) and wb.shape == (g, 2, kq)
    masked = np.array([64, 0, 17], np.int32)
    r1, w1 = oue.ref_masked_ue8m0(a, wa, b, wb, masked)
    r2, w2 = oracle.ref_masked(a, fa, b, fb, masked)
    assert np.array_equal(w1, w2) and np.array_equal(r1[w1], r2[w2])
    a2 = a.reshape(g * mm, k)
    mi = np.repeat(np.array([0, -1, 2], np.int32), mm)
    wa2 = _pack_test_side(ea[0][:, :1].repeat(g * mm, axis=1), axis=0)
    fa2 = np.ldexp(1.0, ea[0][:, :1].repeat(g * mm, axis=1).astype(int) - 127)
    r3, w3 = oue.ref_contiguous_ue8m0(a2, wa2, b, wb, mi)
    r4, w4 = oracle.ref_contiguous(a2, fa2, b, fb, mi)
    assert np.array_equal(w3, w4) and np.array_equal(r3[w3], r4[w4])


def test_ue8m0_planted_byte_order_mistake_is_caught():
    words = np.array([[0x01020304]], np.int32)
    good = oue.unpack_ue8m0(words, 4, axis=1)
    assert list(good[0]) == [4, 3, 2, 1]
    bad = good[:, ::-1]  # big-endian reading
    assert not np.array_equal(bad, np.ascontiguousarray(words).view(np.uint8).reshape(1, 4))


# ----------------------------------------------------------------- K-grouped

def _kg_case(seed, ks, m=40, n=136):
    rng = np.random.default_rng(seed)
    k = int(sum(ks))
    xa = rng.standard_normal((m, k), dtype=np.float32)
    xb = rng.standard_normal((n, k), dtype=np.float32)
    a, sa = quantize_per_row_block(xa)
    b, sb = quantize_per_block(xb)
    c = rng.standard_normal((len(ks), m, n)).astype(np.float32)
    return a, sf_to_mn_major(sa), b, sb, c


def test_k_grouped_sums_to_dense_over_all_k():
    ks = [256, 0, 384, 128]
    a, sfa, b, sfb, _ = _kg_case(3, ks)
    d = okg.ref_k_grouped(a, sfa, b, sfb, ks)
    full = oracle.ref_dense(a, sfa, b, sfb)
    assert np.allclose(d.sum(axis=0), full, rtol=1e-12, atol=1e-9)
    assert not d[1].any()  # empty group contributes exactly zero


def test_k_grouped_single_group_equals_dense_and_c_added_once():
    ks = [512]
    a, sfa, b, sfb, c = _kg_case(4, ks)
    d = okg.ref_k_grouped(a, sfa, b, sfb, ks, c=c)
    assert np.array_equal(d[0], oracle.ref_dense(a, sfa, b, sfb, c=c[0]))
    ks2 = [0, 0]
    a2 = np.zeros((40, 0), np.uint8)
    b2 = np.zeros((136, 0), np.uint8)
    c2 = c[:1].repeat(2, axis=0)
    d2 = okg.ref_k_grouped(a2, np.zeros((0, 40), np.float32), b2, np.zeros((2, 0), np.float32), ks2, c=c2)
    assert np.array_equal(d2, c2.astype(np.float64))


def test_k_grouped_brute_force():
    ks = [128, 256]
    a, sfa, b, sfb, c = _kg_case(5, ks, m=3, n=4)
    d = okg.ref_k_grouped(a, sfa, b, sfb, ks, c=c)
    va, vb = _exact_e4m3(a), _exact_e4m3(b)
    off = [0, 128]
    for g in range(2):
        for i in range(3):
            for j in range(4):
                s = Fraction(float(c[g, i, j]))
                for kk in range(off[g], off[g] + ks[g]):
                    s += va[i, kk] * Fraction(float(sfa[kk // 128, i])) * vb[j, kk] * Fraction(float(sfb[0, kk // 128]))
                assert d[g, i, j] == pytest.approx(float(s), rel=1e-12, abs=1e-12)


def test_k_grouped_planted_offset_mistake_is_caught():
    ks = [128, 256]
    a, sfa, b, sfb, _ = _kg_case(6, ks)
    good = okg.ref_k_grouped(a, sfa, b, sfb, ks)
    # a planted inclusive prefix sum (group g starts at its own end) differs
    bad_off = np.cumsum(ks)
    g = 0
    k0 = int(bad_off[g]) % a.shape[1]
    bad = oracle.ref_dense(a[:, k0:k0 + 128], sfa[k0 // 128:k0 // 128 + 1], b[:, k0:k0 + 128],
                           sfb[:, k0 // 128:k0 // 128 + 1])
    assert not np.allclose(bad, good[0])


# -------------------------------------------------------------- quantization

def _midpoint_probe_values():
    vals = oracle.E4M3_TABLE[:0x7F]  # 0 .. 448, increasing
    mids = (vals[:-1] + vals[1:]) / 2
    f32 = np.concatenate([vals, mids]).astype(np.float32)
    up = np.nextafter(f32, np.float32(np.inf))
    dn = np.nextafter(f32, np.float32(0))
    allv = np.concatenate([f32, up, dn])
    allv = allv[np.abs(allv) <= 448]
    return np.concatenate([allv, -allv, np.array([-0.0], np.float32)])


def test_e4m3_rounding_matches_torch_cast_at_every_midpoint():
    y = _midpoint_probe_values()
    got = oq.e4m3_encode_rne(y)
    want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)
    rng = np.random.default_rng(7)
    r = (rng.standard_normal(200000) * rng.choice([1e-3, 1e-1, 1, 30, 300], 200000)).astype(np.float32)
    r = np.clip(r, -448, 448)
    assert np.array_equal(oq.e4m3_encode_rne(r), torch.from_numpy(r).to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_e4m3_encode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = oracle.E4M3_TABLE[codes].astype(np.float32)
    assert np.array_equal(oq.e4m3_encode_rne(vals), codes)


def test_quant_per_token_matches_torch_based_quantizer():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((37, 512), dtype=np.float32) * np.float32(3.0)
    x[5, 128:256] = 0  # an all-zero block: scale 1, codes 0
    codes, sf = oq.quant_per_token(x)
    want_codes, want_s = quantize_per_row_block(x)
    assert np.array_equal(codes, want_codes)
    assert np.array_equal(sf, sf_to_mn_major(want_s))
    assert sf[1, 5] == 1.0 and not codes[5, 128:256].any()


def test_quant_per_block_matches_torch_based_quantizer():
    rng = np.random.default_rng(9)
    w = rng.standard_normal((300, 384), dtype=np.float32)
    codes, sf = oq.quant_per_block(w)
    want_codes, want_s = quantize_per_block(w)
    assert np.array_equal(codes, want_codes) and np.array_equal(sf, want_s)


def test_quant_scale_rule_and_error_bound():
    rng = np.random.default_rng(10)
    x = (rng.standard_normal((16, 256)) * np.exp(rng.uniform(-8, 8, (16, 1)))).astype(np.float32)
    codes, sf = oq.quant_per_token(x)
    s = sf[:, :16].T  # [M, KB]
    deq = oracle.E4M3_TABLE[codes].reshape(16, 2, 128) * s[..., None].astype(np.float64)
    xb = x.reshape(16, 2, 128).astype(np.float64)
    # the largest magnitude of each block maps to +-448
    amax_idx = np.abs(xb).argmax(axis=-1)
    top = np.take_along_axis(codes.reshape(16, 2, 128), amax_idx[..., None], -1)[..., 0]
    assert set(np.unique(top & 0x7F)) == {0x7E}
    # rounding error: half an E4M3 step (relative 2^-4 in the normal range, 2^-10 * s below it) + FP32 slop
    bound = np.maximum(np.abs(xb) * 2.0 ** -4, s[..., None] * 2.0 ** -10) * (1 + 1e-6)
    assert (np.abs(deq - xb) <= bound).all()


def test_quant_ue8m0_scales_are_minimal_powers_of_two():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((9, 640)) * np.exp(rng.uniform(-6, 6, (9, 1)))).astype(np.float32)
    x[2, :128] = 0
    codes, words = oq.quant_per_token(x, ue8m0=True)
    e = oue.unpack_ue8m0(words, 5, axis=0)[:, :9].T.astype(np.int64)  # [M, KB]
    amax = np.abs(x.reshape(9, 5, 128)).max(-1)
    t = (amax / np.float32(448)).astype(np.float32).astype(np.float64)
    s = np.ldexp(1.0, e - 127)
    nz = amax > 0
    assert (s[nz] >= t[nz]).all() and (s[nz] / 2 < t[nz]).all()
    assert e[2, 0] == 127 and not codes[2, :128].any()
    # power-of-two scaling never needs the clamp: every quotient is within +-448 already
    y = x.reshape(9, 5, 128) / s[..., None]
    assert (np.abs(y) <= 448).all()
    deq = oracle.E4M3_TABLE[codes].reshape(9, 5, 128) * s[..., None]
    bound = np.maximum(np.abs(x.reshape(9, 5, 128)) * 2.0 ** -4, s[..., None] * 2.0 ** -10) * (1 + 1e-6)
    assert (np.abs(deq - x.reshape(9, 5, 128)) <= bound).all()
    # per-block UE8M0 words decode to the same powers of two the codes were scaled by
    cw, ww = oq.quant_per_block(x, ue8m0=True)
    eb = oue.unpack_ue8m0(ww, 5, axis=1)
    amax_b = np.abs(x.reshape(9, 5, 128)).max(axis=(0, 2))
    tb = (amax_b / np.float32(448)).astype(np.float32).astype(np.float64)
    sb = np.ldexp(1.0, eb[0].astype(np.int64) - 127)
    assert (sb >= tb).all() and (sb / 2 < tb).all()


def test_quant_planted_mistakes_are_caught():
    # ties to the odd code, or truncation, disagree with torch on midpoints
    y = _midpoint_probe_values()
    want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mag = np.abs(y).astype(np.float64)
    vals = oracle.E4M3_TABLE[:0x7F]
    trunc = (np.searchsorted(vals, mag, side="right") - 1).astype(np.uint8) | np.where(np.signbit(y), 0x80, 0).astype(np.uint8)
    assert not np.array_equal(trunc, want)


# ---------------------------------------------------------------- MQA logits

def _mqa_case(seed, s=4, s_kv=7, h=3, d=32):
    rng = np.random.default_rng(seed)
    q = torch.from_numpy(rng.standard_normal((s, h, d), dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    kv = torch.from_numpy(rng.standard_normal((s_kv, d), dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    sf = rng.uniform(0.5, 2.0, s_kv).astype(np.float32)
    w = rng.standard_normal((s, h)).astype(np.float32)
    ks = np.array([0, 2, 5, -3][:s], np.int32)
    ke = np.array([7, 5, 5, 100][:s], np.int32)
    return q, kv, sf, w, ks, ke


def test_mqa_brute_force_with_empty_and_clamped_ranges():
    q, kv, sf, w, ks, ke = _mqa_case(12)
    out = omqa.ref_mqa_logits(q, kv, sf, w, ks, ke, clean_logits=True)
    vq, vk = _exact_e4m3(q), _exact_e4m3(kv)
    for i in range(4):
        lo, hi = min(max(ks[i], 0), 7), min(max(ke[i], 0), 7)
        for j in range(7):
            if not (lo <= j < hi):
                assert out[i, j] == -np.inf
                continue
            tot = Fraction(0)
            for hh in range(3):
                dot = sum(vq[i, hh, dd] * vk[j, dd] for dd in range(32)) * Fraction(float(sf[j]))
                tot += max(dot, Fraction(0)) * Fraction(float(w[i, hh]))
            assert out[i, j] == pytest.approx(float(tot), rel=1e-12, abs=1e-12)
    assert np.isneginf(out[2]).all()  # empty range: nothing written, all -inf


def test_mqa_relu_placement_weights_linearity_and_untouched_marking():
    q, kv, sf, w, ks, ke = _mqa_case(13)
    base = omqa.ref_mqa_logits(q, kv, sf, w, ks, ke, clean_logits=False)
    # untouched positions are marked NaN without clean_logits
    assert np.isnan(base[2]).all() and np.isnan(base[1, :2]).all() and np.isfinite(base[0]).all()
    # doubling the weights doubles every written logit
    dbl = omqa.ref_mqa_logits(q, kv, sf, 2 * w, ks, ke, clean_logits=False)
    fin = np.isfinite(base)
    assert np.array_equal(dbl[fin], 2 * base[fin])
    # negating kv moves every head's dot product to the other side of the ReLU:
    # out(kv) + out(-kv) = sum_h w * |dot|, which differs from out(kv) - out(-kv) = sum_h w * dot
    neg = omqa.ref_mqa_logits(q, kv ^ np.uint8(0x80), sf, w, ks, ke, clean_logits=False)
    qd = oracle.decode_e4m3(q)
    kd = oracle.decode_e4m3(kv) * sf[:, None].astype(np.float64)
    dots = np.einsum("ihd,jd->ijh", qd, kd)
    want_abs = (np.abs(dots) * w[:, None, :]).sum(-1)
    want_lin = (dots * w[:, None, :]).sum(-1)
    assert np.allclose((base + neg)[fin], want_abs[fin], rtol=1e-12, atol=1e-12)
    assert np.allclose((base - neg)[fin], want_lin[fin], rtol=1e-12, atol=1e-12)
    # a planted "no ReLU" oracle would give base + neg == 0 instead
    assert not np.allclose((want_lin + (-want_lin))[fin], want_abs[fin])


def test_k_grouped_ue8m0_equals_fp32_form_of_the_same_powers_of_two():
    """Packed UE8M0 words along the global K blocks (a word may hold blocks of two
    groups: ks = 128 + 384 + 0 + 256 puts group boundaries inside words) decode to
    the same K-grouped GEMM as the FP32 scales they were packed from."""
    from workloads.gen import _draw, pack_ue8m0, quantize_per_block, quantize_per_row_block, sf_to_mn_major

    rng = np.random.default_rng(71)
    m, n = 9, 200
    ks = np.array([128, 384, 0, 256], np.int32)
    k = int(ks.sum())
    a, a_s = quantize_per_row_block(_draw(rng, (m, k)), True)
    b, b_s = quantize_per_block(_draw(rng, (n, k)), True)
    c = _draw(rng, (4, m, n))
    sfa = sf_to_mn_major(a_s)
    fp32 = oracle.ref_k_grouped(a, sfa, b, b_s, ks, c)
    words_a = pack_ue8m0(np.where(np.arange(sfa.shape[1]) < m, sfa, 1.0), axis=0)
    ue = oracle.ref_k_grouped_ue8m0(a, words_a, b, pack_ue8m0(b_s, axis=1), ks, c)
    assert np.array_equal(fp32, ue)
    # and a scale moved to the neighbouring byte (a per-group word restart) would not
    bad = words_a.copy().view(np.uint32)
    bad[0] = ((bad[0] << 8) | 127) & 0xFFFFFFFF
    assert not np.array_equal(oracle.ref_k_grouped_ue8m0(a, bad.view(np.int32), b, pack_ue8m0(b_s, axis=1), ks, c),
                              fp32)
