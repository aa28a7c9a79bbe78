"""GPU parity of the weighted-ReLU MQA logits kernel against the FP64 oracle
(``oracle/mqa.py``).  Written logits must meet the GEMM bar (per element
|out - ref| <= 2^-7 |ref| + 1e-3 rms(ref), 1 - cos <= 1e-5); positions outside
each query's key range must be exactly -inf with clean_logits and keep the
caller's bits without it."""

import numpy as np
import pytest
import torch

import oracle
from workloads import gen_mqa

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():  # pragma: no cover - GPU only
    import moe_grouped_gemm_tiles_amd as dg
    from tests._gpu_harness import SENT_F32, note, to_dev


def _run(x, clean, rows_out=None):
    s, s_kv = x["s"], x["s_kv"]
    out = torch.full((s, s_kv), SENT_F32, dtype=torch.int32, device="cuda:0").view(torch.float32)
    dg.fp8_mqa_logits(to_dev(x["q"]).view(torch.float8_e4m3fn),
                      (to_dev(x["kv"]).view(torch.float8_e4m3fn), to_dev(x["sf"])),
                      to_dev(x["w"]), to_dev(x["ks"]), to_dev(x["ke"]), clean, out)
    torch.cuda.synchronize()
    return out


def _check(x, out, clean, rows=None, what=""):
    ref = oracle.ref_mqa_logits(x["q"], x["kv"], x["sf"], x["w"], x["ks"], x["ke"], clean, rows=rows)
    got = out.cpu().numpy() if rows is None else out[torch.as_tensor(rows, device=out.device)].cpu().numpy()
    fin = np.isfinite(ref)
    if clean:
        assert np.isneginf(got[~fin]).all(), f"{what}: positions outside the ranges must be -inf"
    else:
        assert (got[~fin].view(np.int32) == np.int32(SENT_F32)).all(), f"{what}: untouched positions were written"
    rep = oracle.assert_close(got[fin].astype(np.float64), ref[fin], what)
    note(f"{what}: worst={rep['worst_ratio']:.3f} cos_dist={rep['cos_dist']:.2e} written={fin.sum()}")


@pytest.mark.parametrize("clean", [True, False])
@pytest.mark.parametrize("h", [64, 16])
def test_mqa_random_ranges(clean, h):
    x = gen_mqa(70, 300, h, 128, seed=160 + h, ranges="random")  # partial key tile, empty and clamped ranges
    _check(x, _run(x, clean), clean, what=f"mqa random H={h} clean={clean}")


@pytest.mark.parametrize("h", [32, 48])
def test_mqa_head_counts(h):
    x = gen_mqa(40, 260, h, 128, seed=170 + h, ranges="random")
    _check(x, _run(x, True), True, what=f"mqa H={h}")


@pytest.mark.parametrize("s_kv", [200, 100, 129])
def test_mqa_one_partial_key_tile(s_kv):
    """Fewer keys than one workgroup tile: its later key fragments hold rows past S_kv
    (loaded as zeros, never stored), with and without -inf cleaning."""
    x = gen_mqa(33, s_kv, 64, 128, seed=175 + s_kv, ranges="random")
    for clean in (True, False):
        _check(x, _run(x, clean), clean, what=f"mqa S_kv={s_kv} clean={clean}")


def test_mqa_causal_prefill():
    x = gen_mqa(512, 1024, 64, 128, seed=180, ranges="causal")
    _check(x, _run(x, True), True, what="mqa causal S=512 S_kv=1024")


def test_mqa_full_size_sampled():
    """The benchmark's shape: 4096 queries, 8192 keys (causal with a 4096-key prefix), 64 heads."""
    x = gen_mqa(4096, 8192, 64, 128, seed=181, ranges="causal")
    out = _run(x, True)
    rng = np.random.default_rng(182)
    rows = np.unique(np.concatenate([[0, 4095], rng.choice(4096, 24, replace=False)]))
    _check(x, out, True, rows=rows, what="mqa full size (sampled rows)")
    assert not torch.isnan(out).any()
