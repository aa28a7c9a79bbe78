"""GPU parity tests: the HIP library (called through its C ABI via the
binding) against the FP64 CPU oracle on seeded inputs.

Bar: per element |D - ref| <= 2^-7 |ref| + 1e-3 rms(ref), 1 - cos <= 1e-5,
no NaN/Inf in outputs; bit-exact where the result is exactly representable
(one-hot products, E4M3 decode); rows the library must not write are
compared bit-for-bit with the sentinel they were filled with.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import gen_contiguous, gen_dense, gen_masked, sf_aligned_size

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():  # pragma: no cover - GPU only
    from tests._gpu_harness import (as_f64, fp8_dev, note, out_buffer, raw_bits, run_contiguous, run_dense,
                                    run_masked, sentinel_of, to_dev)
    import moe_grouped_gemm_tiles_amd as dg


def _check_dense(x, d, what):
    ref = oracle.ref_dense(x["a"], x["sfa"], x["b"], x["sfb"], x.get("c"))
    rep = oracle.assert_close(as_f64(d), ref, what)
    note(f"{what}: worst={rep['worst_ratio']:.3f} cos_dist={rep['cos_dist']:.2e}")


def test_e4m3_decode_all_codes_on_gpu():
    """Every E4M3 code through the matrix core equals the oracle's closed-form value (FP32 out)."""
    m, n, k = 256, 16, 128
    a = np.zeros((m, k), np.uint8)
    a[:, 0] = np.arange(256, dtype=np.uint8)
    b = np.zeros((n, k), np.uint8)
    b[:, 0] = 0x38  # 1.0
    sfa = np.ones((1, m), np.float32)
    sfb = np.ones((1, 1), np.float32)
    d = out_buffer((m,), n, "fp32")
    dg.fp8_gemm_nt((fp8_dev(a), to_dev(sfa)), (fp8_dev(b), to_dev(sfb)), d)
    torch.cuda.synchronize()
    got = d.cpu().numpy().astype(np.float64)
    want = np.repeat(oracle.E4M3_TABLE[:, None], n, axis=1)
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all()
    assert np.array_equal(got[~nan], want[~nan])


@pytest.mark.parametrize("pow2,out", [(False, "bf16"), (True, "bf16"), (True, "fp32")])
def test_one_hot_bit_exact(pow2, out):
    """A row m is one-hot at k = perm[m]: D[m, n] = B[n, perm[m]] * scales, exactly (pins lane maps and swizzle)."""
    rng = np.random.default_rng(50)
    m, n, k = 256, 384, 512
    perm = rng.permutation(k)[:m]
    a = np.zeros((m, k), np.uint8)
    a[np.arange(m), perm] = 0x38
    b = rng.integers(0, 256, (n, k), dtype=np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x40
    kb, nb = k // 128, n // 128
    ea = rng.integers(-3, 4, (kb, m)) if pow2 else np.zeros((kb, m), int)
    eb = rng.integers(-3, 4, (nb, kb)) if pow2 else np.zeros((nb, kb), int)
    x = dict(m=m, n=n, k=k, out_dtype=out, a=a, b=b, c=None,
             sfa=np.ldexp(1.0, ea).astype(np.float32), sfb=np.ldexp(1.0, eb).astype(np.float32))
    d = run_dense(x)
    ref = oracle.ref_dense(a, x["sfa"], b, x["sfb"])
    want = torch.from_numpy(ref).to(torch.bfloat16 if out == "bf16" else torch.float32)
    assert torch.equal(d.cpu().view(torch.int16 if out == "bf16" else torch.int32),
                       want.view(torch.int16 if out == "bf16" else torch.int32))


def test_dense_small_config():
    x = gen_dense(128, 256, 512, seed=0)
    _check_dense(x, run_dense(x), "dense M=128 N=256 K=512")


@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (17, 40, 256), (130, 200, 384), (300, 136, 128),
                                   (64, 2112, 1024), (257, 520, 640), (129, 264, 1152)])
def test_dense_ragged_shapes(m, n, k):
    x = gen_dense(m, n, k, seed=m + n + k)
    ld = -(-n // 8) * 8 + 8  # padded leading dimension
    d = run_dense(x, ld_d=ld)
    _check_dense(x, d, f"dense ragged M={m} N={n} K={k}")


@pytest.mark.parametrize("m,n,k,fmt", [(300, 1005, 256, "fp32"), (300, 13, 384, "fp32"), (520, 2110, 512, "fp32"),
                                       (300, 1005, 256, "ue8m0"), (260, 229, 384, "fp32")])
def test_dense_bf16_ragged_n_columns(m, n, k, fmt):
    """BF16 output with N not a multiple of 8 (16-byte stores of eight columns fall back
    to element stores at the edge) and a padded leading dimension: values match the
    oracle and the padding columns past N keep the sentinel."""
    ld = (n + 7) // 8 * 8 + 8
    x = gen_dense(m, n, k, seed=7 * n + k, scale_fmt=fmt)
    d = run_dense(x, ld_d=ld)
    ref = (oracle.ref_dense_ue8m0 if fmt == "ue8m0" else oracle.ref_dense)(x["a"], x["sfa"], x["b"], x["sfb"])
    oracle.assert_close(as_f64(d), ref, f"bf16 ragged N m={m} n={n} k={k} {fmt}")
    full = d.as_strided((m, ld), (ld, 1))  # d is the first n columns of an [m, ld] buffer
    assert (raw_bits(full)[:, n:] == sentinel_of(d)).all(), "columns past N were written"


def test_dense_padded_sfa_and_k_zero():
    x = gen_dense(70, 64, 256, seed=3, ld_sfa=96)
    x["sfa"][:, 70:] = np.nan  # padding columns must never be read into valid rows
    _check_dense(x, run_dense(x), "dense padded ld_sfa")
    # K == 0: D = C (FP32), or 0 without C
    c = np.random.default_rng(1).standard_normal((33, 40)).astype(np.float32)
    y = dict(m=33, n=40, k=0, out_dtype="fp32", a=np.zeros((33, 0), np.uint8), b=np.zeros((40, 0), np.uint8),
             sfa=np.zeros((0, 36), np.float32), sfb=np.zeros((1, 0), np.float32), c=c)
    d = out_buffer((33,), 40, "fp32")
    dg.fp8_gemm_nt((fp8_dev(y["a"]), to_dev(y["sfa"])), (fp8_dev(y["b"]), to_dev(y["sfb"])), d,
                   to_dev(c))
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy(), c)


@pytest.mark.parametrize("out", ["fp32", "bf16"])
def test_dense_with_c(out):
    x = gen_dense(200, 300, 512, seed=8, with_c=True, out_dtype=out)
    _check_dense(x, run_dense(x, ld_d=304), f"dense+C {out}")
    d2 = run_dense(x, ld_d=304, c_in_place=True)
    _check_dense(x, d2, f"dense+C in place {out}")


def test_zero_a_gives_c_exactly():
    x = gen_dense(96, 128, 256, seed=9, with_c=True, out_dtype="fp32")
    x["a"][:] = 0
    d = run_dense(x)
    assert np.array_equal(d.cpu().numpy(), x["c"])
    y = gen_dense(96, 128, 256, seed=9)
    y["a"][:] = 0
    d = run_dense(y)
    assert not d.float().cpu().numpy().any()


def test_single_slab_isolation():
    x = gen_dense(160, 272, 640, seed=10)
    for j in range(5):
        y = dict(x)
        y["sfa"] = x["sfa"].copy()
        y["sfa"][np.arange(5) != j] = 0
        _check_dense(y, run_dense(y), f"single slab {j}")


def test_determinism():
    x = gen_dense(512, 1024, 2048, seed=12)
    d1 = raw_bits(run_dense(x))
    d2 = raw_bits(run_dense(x))
    assert np.array_equal(d1, d2)


def _check_contiguous(x, d, what):
    ref, written = oracle.ref_contiguous(x["a"], x["sfa"], x["b"], x["sfb"], x["m_indices"])
    got = as_f64(d)
    rep = oracle.assert_close(got[written], ref[written], what)
    bits = raw_bits(d)
    assert (bits[~written] == sentinel_of(d)).all(), f"{what}: padding rows were written"
    note(f"{what}: worst={rep['worst_ratio']:.3f} cos_dist={rep['cos_dist']:.2e} rows={written.sum()}")


@pytest.mark.parametrize("sizes", [[130, 1, 0, 255], [128, 128], [5]])
def test_contiguous_small(sizes):
    x = gen_contiguous(len(sizes), 320, 512, seed=20 + len(sizes), m_sizes=sizes)
    _check_contiguous(x, run_contiguous(x), f"contiguous sizes={sizes}")


def test_contiguous_bad_group_ids_are_skipped():
    x = gen_contiguous(3, 256, 256, seed=22, m_sizes=[100, 200, 50])
    mi = x["m_indices"].copy()
    mi[256:384] = 7  # out-of-range group id on a whole block: skipped, not written
    x["m_indices"] = mi
    d = run_contiguous(x)
    bits = raw_bits(d)
    assert (bits[256:384] == sentinel_of(d)).all()
    ref, written = oracle.ref_contiguous(x["a"], x["sfa"], x["b"], x["sfb"], mi)
    oracle.assert_close(as_f64(d)[written], ref[written], "contiguous with bad ids")


def test_contiguous_equals_dense_per_group():
    x = gen_contiguous(3, 384, 512, seed=24, m_sizes=[256, 128, 384])
    dc = as_f64(run_contiguous(x))
    off = 0
    for g, s in enumerate(x["m_sizes"]):
        rows = slice(off, off + int(s))
        y = dict(m=int(s), n=384, k=512, out_dtype="bf16", a=x["a"][rows],
                 sfa=np.ascontiguousarray(x["sfa"][:, rows]), b=x["b"][g], sfb=x["sfb"][g], c=None)
        dd = as_f64(run_dense(y))
        oracle.assert_close(dc[rows], dd, f"group {g} contiguous vs dense")
        off += int(s)


def _check_masked(x, d, what):
    ref, written = oracle.ref_masked(x["a"], x["sfa"], x["b"], x["sfb"], x["masked_m"])
    got = as_f64(d)
    rep = oracle.assert_close(got[written], ref[written], what)
    bits = raw_bits(d)
    assert (bits[~written] == sentinel_of(d)).all(), f"{what}: masked rows were written"
    note(f"{what}: worst={rep['worst_ratio']:.3f} cos_dist={rep['cos_dist']:.2e} rows={written.sum()}")


@pytest.mark.parametrize("poison", [False, True])
def test_masked_small(poison):
    x = gen_masked(5, 200, 384, 256, seed=33, masked_m=[0, 200, 64, 1, 300], poison=poison)
    _check_masked(x, run_masked(x, expected_m=100), f"masked poison={poison}")


def test_masked_all_empty():
    x = gen_masked(3, 64, 128, 128, seed=34, masked_m=[0, -5, 0])
    d = run_masked(x)
    assert (raw_bits(d) == sentinel_of(d)).all()


def test_masked_fp32_out():
    x = gen_masked(4, 96, 160, 384, seed=35, masked_m=[96, 50, 3, 17], out_dtype="fp32")
    _check_masked(x, run_masked(x), "masked fp32")


def test_masked_narrow_n():
    """N <= 128 takes the 128x128 masked tiles (wider N takes the 256-row tiles)."""
    x = gen_masked(4, 272, 128, 512, seed=37, masked_m=[272, 129, 0, 5])
    _check_masked(x, run_masked(x, expected_m=64), "masked n=128")


def test_num_cus_cap_gives_same_bits():
    x = gen_dense(640, 768, 1024, seed=36)
    ref_bits = raw_bits(run_dense(x))
    try:
        dg.set_num_cus(7)
        assert np.array_equal(raw_bits(run_dense(x)), ref_bits)
    finally:
        dg.set_num_cus(0)


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_contiguous_ragged_last_round_split(fmt):
    """Capped at 4 CUs, 1280 rows (5 row tiles of 256) x 2 column tiles leave a
    last round of 2 tiles in 4 slots, so rows 1024.. go to a second launch of
    128x128 tiles; the split cuts through group 1.  The bits must equal the
    uncapped call (one round, one launch) and the oracle."""
    x = gen_contiguous(3, 512, 512, seed=38, m_sizes=[300, 700, 100], scale_fmt=fmt)
    assert x["m_total"] == 1280
    whole = run_contiguous(x)
    try:
        dg.set_num_cus(4)
        split = run_contiguous(x)
    finally:
        dg.set_num_cus(0)
    assert np.array_equal(raw_bits(split), raw_bits(whole))
    ref_fn = oracle.ref_contiguous if fmt == "fp32" else oracle.ref_contiguous_ue8m0
    ref, written = ref_fn(x["a"], x["sfa"], x["b"], x["sfb"], x["m_indices"])
    oracle.assert_close(as_f64(split)[written], ref[written], f"contiguous tail split {fmt}")
    assert (raw_bits(split)[~written] == sentinel_of(split)).all()


@pytest.mark.parametrize("m,out", [(48, "fp32"), (128, "bf16"), (100, "fp32")])
def test_dense_split_k_with_c(m, out):
    """Skinny M takes the split-K path (FP32 partials, ordered in-kernel reduction); C is added once."""
    x = gen_dense(m, 520, 2048, seed=60 + m, with_c=True, out_dtype=out)
    _check_dense(x, run_dense(x, ld_d=528), f"split-K + C M={m} {out}")


def test_split_k_determinism_and_sentinel_columns():
    x = gen_dense(64, 2112, 7168, seed=61)
    d1 = run_dense(x, ld_d=2120)
    d2 = run_dense(x, ld_d=2120)
    assert np.array_equal(raw_bits(d1), raw_bits(d2))
    _check_dense(x, d1, "split-K M=64 N=2112 K=7168")


def test_split_k_threads_sharing_a_stream():
    """Two host threads issue skinny (split-K) calls of different shapes on one stream,
    each call with the workspace the binding takes from torch's allocator: every output
    equals the single-threaded result."""
    import threading

    xs = [gen_dense(64, 2112, 7168, seed=70), gen_dense(100, 1040, 4096, seed=71)]
    want = [raw_bits(run_dense(x)) for x in xs]
    dev = [(fp8_dev(x["a"]), to_dev(x["sfa"]), fp8_dev(x["b"]), to_dev(x["sfb"])) for x in xs]
    s = torch.cuda.Stream()
    calls = 24
    outs = [[out_buffer((x["m"],), x["n"], x["out_dtype"]) for _ in range(calls)] for x in xs]
    torch.cuda.synchronize()  # inputs and sentinel fills are on the default stream
    start = threading.Barrier(2)
    errors = []

    def worker(i):
        try:
            a, sfa, b, sfb = dev[i]
            start.wait()
            with torch.cuda.stream(s):
                for d in outs[i]:
                    dg.fp8_gemm_nt((a, sfa), (b, sfb), d)
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        for j, d in enumerate(outs[i]):
            assert np.array_equal(raw_bits(d), want[i]), f"input {i}, call {j}"
