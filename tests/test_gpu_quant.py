"""GPU parity of the FP8 quantization kernels against the oracle's cast
(``oracle/quant.py``): codes and scales must match bit for bit, since both
sides take the same FP32 steps (FP32 scale, correctly rounded FP32 quotient)
and then decide the E4M3 code (round to nearest, ties to even)."""

import numpy as np
import pytest
import torch

import oracle
from workloads import gen_quant_input

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():  # pragma: no cover - GPU only
    import moe_grouped_gemm_tiles_amd as dg
    from tests._gpu_harness import note, to_dev


def _x_dev(x, dtype):
    t = to_dev(x.astype(np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _run_token(x, dtype, ue, ld=None):
    m, k = x.shape
    ld = (m + 3) // 4 * 4 if ld is None else ld
    xd = _x_dev(x, dtype)
    q = torch.full((m, k), 0xAA, dtype=torch.uint8, device="cuda:0")
    kr = ((k // 128 + 3) // 4) if ue else k // 128
    sf = torch.full((kr, ld), -7, dtype=torch.int32, device="cuda:0")
    if not ue:
        sf = sf.view(torch.float32)
    dg.per_token_cast_to_fp8(xd, q, sf)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sf.cpu().numpy()


def _run_block(w, dtype, ue):
    n, k = w.shape
    wd = _x_dev(w, dtype)
    q = torch.full((n, k), 0xAA, dtype=torch.uint8, device="cuda:0")
    kr = ((k // 128 + 3) // 4) if ue else k // 128
    sf = torch.full(((n + 127) // 128, kr), -7, dtype=torch.int32, device="cuda:0")
    if not ue:
        sf = sf.view(torch.float32)
    dg.per_block_cast_to_fp8(wd, q, sf)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sf.cpu().numpy()


def _probe_rows():
    """Rows whose 128-blocks each hold 448 (so s = 1 and x / s = x) and, elsewhere,
    every E4M3 value, every midpoint and the FP32 neighbours of both."""
    vals = oracle.E4M3_TABLE[:0x7F]
    mids = (vals[:-1] + vals[1:]) / 2
    f32 = np.concatenate([vals, mids]).astype(np.float32)
    probe = np.concatenate([f32, np.nextafter(f32, np.float32(np.inf)), np.nextafter(f32, np.float32(0))])
    probe = probe[np.abs(probe) <= 448]
    probe = np.concatenate([probe, -probe, np.array([-0.0], np.float32)])
    per = 127
    nblk = -(-len(probe) // per)
    probe = np.concatenate([probe, np.zeros(nblk * per - len(probe), np.float32)])
    rows = np.zeros((nblk, 128), np.float32)
    rows[:, 0] = 448
    rows[:, 1:] = probe.reshape(nblk, per)
    k = 640
    pad = (-nblk) % (k // 128)
    rows = np.concatenate([rows, np.tile(rows[:1], (pad, 1))])
    return rows.reshape(-1, k)


def test_rounding_of_every_code_midpoint_and_neighbour():
    x = _probe_rows()
    q, sf = _run_token(x, "fp32", ue=False)
    want_q, want_sf = oracle.quant_per_token(x)
    m = x.shape[0]
    assert (sf[:, :m] == 1.0).all()
    assert np.array_equal(q, want_q)
    note(f"{x.size} probe values: codes identical to the oracle")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("ue", [False, True])
def test_per_token_bit_exact(dtype, ue):
    x = gen_quant_input(300, 640, seed=120 + ue, dtype=dtype)  # 5 K-blocks: a partial 4-block tile
    ld = 308
    q, sf = _run_token(x, dtype, ue, ld=ld)
    want_q, want_sf = oracle.quant_per_token(x, ld_sf=ld, ue8m0=ue)
    assert np.array_equal(q, want_q)
    assert np.array_equal(sf[:, :300].view(np.int32), want_sf[:, :300].view(np.int32))
    assert (sf[:, 300:].view(np.int32) == -7).all()  # padding columns are not written
    assert not q[0, 128:256].any()  # the all-zero block


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("ue", [False, True])
def test_per_block_bit_exact(dtype, ue):
    w = gen_quant_input(300, 640, seed=130 + ue, dtype=dtype)  # partial last row block
    q, sf = _run_block(w, dtype, ue)
    want_q, want_sf = oracle.quant_per_block(w, ue8m0=ue)
    assert np.array_equal(q, want_q)
    assert np.array_equal(sf.view(np.int32), want_sf.view(np.int32))


def _extreme_rows(dtype, seed):
    """Rows of N(0,1) values times 2^k, k from denormal inputs to near the FP32 limit and on
    both sides of where the FP32 scale amax/448 leaves [2^-80, 2^100]; in every row some
    values 2^-40 smaller (their quotients round to an E4M3 zero), two -0 and one +0."""
    rng = np.random.default_rng(seed)
    ks = [-133, -120, -100, -75, -74, -73, -72, 0, 100, 105, 106, 107, 108, 124]
    rows = []
    for k in ks:
        for _ in range(2):
            r = rng.standard_normal(512).astype(np.float64) * 2.0 ** k
            tiny = rng.random(512) < 0.05
            r[tiny] *= 2.0 ** -40
            r[rng.integers(0, 512, 2)] = -0.0
            r[rng.integers(0, 512)] = 0.0
            rows.append(r.astype(np.float32))
    x = np.stack(rows)
    if dtype == "bf16":
        x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.isfinite(x).all()
    return x


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_extreme_magnitudes_bit_exact(dtype):
    """Scales far from 1 take the division's general path, the others the one with the
    reciprocal refined per block: both must give the oracle's codes and scales."""
    x = _extreme_rows(dtype, seed=140)
    q, sf = _run_token(x, dtype, ue=False)
    want_q, want_sf = oracle.quant_per_token(x)
    m = x.shape[0]
    assert np.array_equal(sf[:, :m].view(np.int32), want_sf[:, :m].view(np.int32))
    bad = np.argwhere(q != want_q)
    assert bad.size == 0, f"per-token: {len(bad)} codes differ, first at {bad[:3].tolist()}"
    # row blocks (x holds two rows per k, in the order of ks): amax at k = -72 (scale just
    # inside the lower bound), k = -74 (just outside), k = 106 (just inside the upper bound),
    # then a partial block at k = 124 (outside)
    w = np.concatenate([np.resize(x[0:14], (128, 512)), np.resize(x[0:10], (128, 512)),
                        np.resize(x[16:22], (128, 512)), np.resize(x[22:28], (50, 512))])
    qb, sfb = _run_block(w, dtype, ue=False)
    want_qb, want_sfb = oracle.quant_per_block(w)
    assert np.array_equal(sfb.view(np.int32), want_sfb.view(np.int32))
    assert np.array_equal(qb, want_qb), f"per-block: {int((qb != want_qb).sum())} codes differ"


def test_cast_then_gemm_matches_oracle():
    """GPU cast of both operands feeding the GPU GEMM equals the oracle's cast + GEMM."""
    xa = gen_quant_input(256, 1024, seed=140)
    xb = gen_quant_input(384, 1024, seed=141)
    qa, sfa = _run_token(xa, "bf16", ue=False)
    qb, sfb = _run_block(xb, "bf16", ue=False)
    wa, wsa = oracle.quant_per_token(xa)
    wb, wsb = oracle.quant_per_block(xb)
    assert np.array_equal(qa, wa) and np.array_equal(qb, wb)
    d = torch.empty(256, 384, dtype=torch.float32, device="cuda:0")
    dg.fp8_gemm_nt((to_dev(qa).view(torch.float8_e4m3fn), to_dev(sfa)),
                   (to_dev(qb).view(torch.float8_e4m3fn), to_dev(sfb)), d)
    torch.cuda.synchronize()
    oracle.assert_close(d.cpu().numpy().astype(np.float64), oracle.ref_dense(wa, wsa, wb, wsb), "cast + GEMM")


def test_quant_full_size_sampled():
    """The benchmark's shapes: activations [33280, 7168] per token, weights [32768, 7168] per block (BF16)."""
    x = gen_quant_input(33280, 7168, seed=150)
    q, sf = _run_token(x, "bf16", ue=False)
    rng = np.random.default_rng(151)
    rows = np.unique(np.concatenate([[0, 33279], rng.choice(33280, 200, replace=False)]))
    wq, wsf = oracle.quant_per_token(x[rows])
    assert np.array_equal(q[rows], wq)
    assert np.array_equal(sf[:, rows], wsf[:, :len(rows)])
    del x, q
    w = gen_quant_input(32768, 7168, seed=152)
    q, sf = _run_block(w, "bf16", ue=True)
    for nb in (0, 97, 255):
        wq, wsf = oracle.quant_per_block(w[nb * 128:(nb + 1) * 128], ue8m0=True)
        assert np.array_equal(q[nb * 128:(nb + 1) * 128], wq)
        assert np.array_equal(sf[nb], wsf[0])
