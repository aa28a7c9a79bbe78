"""GPU parity of the UE8M0-scale GEMMs, the K-grouped GEMM and the weight-gradient
entry points against the FP64 CPU oracle (library called through its C ABI
via the binding).

Bar as for the FP32-scale GEMMs: per element |D - ref| <= 2^-7 |ref| +
1e-3 rms(ref), 1 - cos <= 1e-5; bit-exact where the result is exactly
representable (one-hot rows with power-of-two scales); unwritten rows keep
their sentinel bit-for-bit.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import gen_contiguous, gen_dense, gen_k_grouped, gen_masked, pack_ue8m0

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():  # pragma: no cover - GPU only
    from tests._gpu_harness import (as_f64, note, raw_bits, run_contiguous, run_dense, run_k_grouped, run_masked,
                                    sentinel_of)


def _check_ue_dense(x, d, what):
    ref = oracle.ref_dense_ue8m0(x["a"], x["sfa"], x["b"], x["sfb"], x.get("c"))
    rep = oracle.assert_close(as_f64(d), ref, what)
    note(f"{what}: worst={rep['worst_ratio']:.3f} cos_dist={rep['cos_dist']:.2e}")


@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_ue8m0_one_hot_bit_exact(out):
    """One-hot A rows select B entries scaled by 2^(ea + eb): exact, so the bits must match."""
    rng = np.random.default_rng(70)
    m, n, k = 256, 272, 640
    perm = rng.permutation(k)[:m]
    a = np.zeros((m, k), np.uint8)
    a[np.arange(m), perm] = 0x38
    b = rng.integers(0, 256, (n, k), dtype=np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x40
    kb, nb = k // 128, 3
    ea = rng.integers(-20, 21, (kb, m))
    eb = rng.integers(-20, 21, (nb, kb))
    sfa = pack_ue8m0(np.ldexp(1.0, ea), axis=0)
    sfb = pack_ue8m0(np.ldexp(1.0, eb), axis=1)
    x = dict(m=m, n=n, k=k, out_dtype=out, a=a, b=b, c=None, sfa=sfa, sfb=sfb)
    d = run_dense(x)
    ref = oracle.ref_dense_ue8m0(a, sfa, b, sfb)
    want = torch.from_numpy(ref).to(torch.bfloat16 if out == "bf16" else torch.float32)
    assert torch.equal(d.cpu().view(torch.int16 if out == "bf16" else torch.int32),
                       want.view(torch.int16 if out == "bf16" else torch.int32))


@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (70, 200, 640), (257, 520, 1152), (300, 136, 2560),
                                   (48, 520, 2048), (128, 2112, 7168)])
def test_ue8m0_dense_shapes(m, n, k):
    """Ragged tiles, K not a multiple of 512 (partial packed word), and the split-K path (M <= 128)."""
    x = gen_dense(m, n, k, seed=71 + m + k, scale_fmt="ue8m0")
    _check_ue_dense(x, run_dense(x, ld_d=-(-n // 8) * 8 + 8), f"ue8m0 dense M={m} N={n} K={k}")


@pytest.mark.parametrize("m,out", [(200, "fp32"), (100, "bf16")])
def test_ue8m0_dense_with_c_and_in_place(m, out):
    x = gen_dense(m, 300, 1024, seed=72 + m, with_c=True, out_dtype=out, scale_fmt="ue8m0")
    _check_ue_dense(x, run_dense(x, ld_d=304), f"ue8m0 dense+C M={m} {out}")
    _check_ue_dense(x, run_dense(x, ld_d=304, c_in_place=True), f"ue8m0 dense+C in place M={m} {out}")


def test_ue8m0_nan_scale_byte_gives_nan_row():
    """Scale byte 255 is NaN: the rows it scales come out NaN, the others do not."""
    x = gen_dense(64, 128, 512, seed=73, out_dtype="fp32", scale_fmt="ue8m0")
    sfa = x["sfa"].view(np.uint8).reshape(x["sfa"].shape[0], -1, 4).copy()
    sfa[0, 5, 2] = 255  # row 5, K block 2
    x["sfa"] = sfa.view(np.int32).reshape(x["sfa"].shape)
    d = run_dense(x).cpu().numpy()
    ref = oracle.ref_dense_ue8m0(x["a"], x["sfa"], x["b"], x["sfb"])
    assert np.isnan(ref[5]).all() and np.isnan(d[5]).all()
    keep = np.arange(64) != 5
    oracle.assert_close(d[keep].astype(np.float64), ref[keep], "ue8m0 rows without the NaN scale")


def test_ue8m0_matches_fp32_path_on_power_of_two_scales():
    """The block-scaled MFMA path and the FP32-promotion path agree on the same powers of two."""
    x = gen_dense(384, 512, 2048, seed=74, out_dtype="fp32", scale_fmt="ue8m0")
    d_ue = as_f64(run_dense(x))
    kb = 2048 // 128
    y = dict(x)
    y["sfa"] = oracle.decode_ue8m0_sf(x["sfa"], kb, 0).astype(np.float32)
    y["sfb"] = oracle.decode_ue8m0_sf(x["sfb"], kb, 1).astype(np.float32)
    d_f = as_f64(run_dense(y))
    oracle.assert_close(d_ue, d_f, "ue8m0 vs fp32 scales")


@pytest.mark.parametrize("sizes", [[130, 1, 0, 255], [128, 384]])
def test_ue8m0_contiguous(sizes):
    x = gen_contiguous(len(sizes), 320, 640, seed=75 + len(sizes), m_sizes=sizes, scale_fmt="ue8m0")
    d = run_contiguous(x)
    ref, written = oracle.ref_contiguous_ue8m0(x["a"], x["sfa"], x["b"], x["sfb"], x["m_indices"])
    oracle.assert_close(as_f64(d)[written], ref[written], f"ue8m0 contiguous {sizes}")
    assert (raw_bits(d)[~written] == sentinel_of(d)).all()


@pytest.mark.parametrize("poison", [False, True])
def test_ue8m0_masked(poison):
    x = gen_masked(5, 200, 384, 1152, seed=77, masked_m=[0, 200, 64, 1, 300], poison=poison, scale_fmt="ue8m0")
    d = run_masked(x, expected_m=100)
    ref, written = oracle.ref_masked_ue8m0(x["a"], x["sfa"], x["b"], x["sfb"], x["masked_m"])
    oracle.assert_close(as_f64(d)[written], ref[written], f"ue8m0 masked poison={poison}")
    assert (raw_bits(d)[~written] == sentinel_of(d)).all()


def _check_kg(x, d, with_c, what):
    ref = oracle.ref_k_grouped(x["a"], x["sfa"], x["b"], x["sfb"], x["ks"], c=x["c"] if with_c else None)
    got = as_f64(d)
    for g in range(x["num_groups"]):
        if x["ks"][g] == 0:
            # an empty group writes exactly C (or zero)
            assert np.array_equal(got[g], ref[g]), f"{what}: empty group {g}"
            continue
        rep = oracle.assert_close(got[g], ref[g], f"{what} group {g}")
        note(f"{what} group {g} (K={x['ks'][g]}): worst={rep['worst_ratio']:.3f} cos_dist={rep['cos_dist']:.2e}")


@pytest.mark.parametrize("with_c", [True, False])
def test_k_grouped_small(with_c):
    x = gen_k_grouped(4, 200, 300, seed=80, ks=[256, 0, 384, 128])
    _check_kg(x, run_k_grouped(x, with_c=with_c), with_c, f"k-grouped c={with_c}")


def test_k_grouped_wgrad_in_place_and_large_tiles():
    x = gen_k_grouped(3, 384, 640, seed=81, ks=[1024, 128, 0])
    _check_kg(x, run_k_grouped(x, in_place=True), True, "k-grouped wgrad in place")


def _check_kg_ue(x, d, with_c, what):
    ref = oracle.ref_k_grouped_ue8m0(x["a"], x["sfa"], x["b"], x["sfb"], x["ks"], c=x["c"] if with_c else None)
    got = as_f64(d)
    for g in range(x["num_groups"]):
        if x["ks"][g] == 0:
            assert np.array_equal(got[g], ref[g]), f"{what}: empty group {g}"
            continue
        rep = oracle.assert_close(got[g], ref[g], f"{what} group {g}")
        note(f"{what} group {g} (K={x['ks'][g]}): worst={rep['worst_ratio']:.3f} cos_dist={rep['cos_dist']:.2e}")


@pytest.mark.parametrize("with_c", [True, False])
def test_k_grouped_ue8m0_small(with_c):
    # 128 + 0 + 384 + 256: group boundaries fall inside packed words
    x = gen_k_grouped(4, 200, 300, seed=84, ks=[128, 0, 384, 256], scale_fmt="ue8m0")
    _check_kg_ue(x, run_k_grouped(x, with_c=with_c), with_c, f"k-grouped ue8m0 c={with_c}")


def test_k_grouped_ue8m0_wgrad_in_place_and_large_tiles():
    x = gen_k_grouped(3, 384, 640, seed=85, ks=[1024, 128, 0], scale_fmt="ue8m0")
    _check_kg_ue(x, run_k_grouped(x, in_place=True), True, "k-grouped ue8m0 wgrad in place")


def test_k_grouped_single_group_equals_dense():
    x = gen_k_grouped(1, 256, 512, seed=82, ks=[1536], with_c=False)
    dk = as_f64(run_k_grouped(x, with_c=False))[0]
    y = dict(m=256, n=512, k=1536, out_dtype="fp32", a=x["a"], sfa=x["sfa"], b=x["b"], sfb=x["sfb"], c=None)
    dd = as_f64(run_dense(y))
    assert np.array_equal(dk, dd)  # same tiles, same slab order -> same bits


def test_dense_wgrad_accumulates_in_place():
    import moe_grouped_gemm_tiles_amd as dg
    from tests._gpu_harness import fp8_dev, to_dev
    x = gen_dense(300, 264, 1024, seed=83, with_c=True, out_dtype="fp32")
    d = to_dev(x["c"])
    dg.wgrad_fp8_gemm_nt((fp8_dev(x["a"]), to_dev(x["sfa"])), (fp8_dev(x["b"]), to_dev(x["sfb"])), d)
    torch.cuda.synchronize()
    ref = oracle.ref_dense(x["a"], x["sfa"], x["b"], x["sfb"], x["c"])
    oracle.assert_close(as_f64(d), ref, "dense wgrad in place")
