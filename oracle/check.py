"""Acceptance check of a GEMM result against the FP64 reference.
TEST INFRASTRUCTURE ONLY.

Bar (fixed for this library; the pages give no tolerance):

* element-wise  |D - ref| <= 2^-7 * |ref| + 1e-3 * rms(ref)   over the checked set;
* 1 - cos(D, ref) <= 1e-5                                     over the checked set;
* no NaN or Inf in a checked element.

Why this leaves room: BF16 round-to-nearest-even contributes at most 2^-9
relative error per element, a quarter of the 2^-7 term; FP32 accumulation
of at most 128 slab partials (K = 16384) adds O(1e-6) relative error; the
rms term absorbs cancellation near zero, where relative error is undefined.
An empty checked set passes (all rows masked), but callers still check the
untouched rows separately.
"""

from __future__ import annotations

import numpy as np

TOL_REL = 2.0 ** -7
TOL_RMS = 1e-3
TOL_COS = 1e-5


def tolerance_report(d, ref) -> dict:
    """Compare result ``d`` with FP64 ``ref`` (same shape; both are flattened)."""
    d = np.asarray(d, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    assert d.shape == ref.shape
    n = d.size
    if n == 0:
        return dict(ok=True, n=0, worst_ratio=0.0, cos_dist=0.0, nonfinite=0, rms=0.0)
    nonfinite = int((~np.isfinite(d)).sum())
    rms = float(np.sqrt(np.mean(ref * ref)))
    bound = TOL_REL * np.abs(ref) + TOL_RMS * rms
    err = np.abs(d - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    worst = float(np.nanmax(ratio)) if nonfinite == 0 else float("inf")
    dd = float(np.dot(d, d)) if nonfinite == 0 else float("nan")
    rr = float(np.dot(ref, ref))
    if nonfinite == 0 and dd > 0 and rr > 0:
        cos_dist = 1.0 - float(np.dot(d, ref)) / np.sqrt(dd * rr)
    elif nonfinite == 0 and dd == 0 and rr == 0:
        cos_dist = 0.0
    else:
        cos_dist = float("inf")
    ok = nonfinite == 0 and worst <= 1.0 and cos_dist <= TOL_COS
    return dict(ok=bool(ok), n=n, worst_ratio=worst, cos_dist=cos_dist, nonfinite=nonfinite, rms=rms)


def assert_close(d, ref, what: str = "") -> dict:
    rep = tolerance_report(d, ref)
    assert rep["ok"], f"{what}: tolerance check failed: {rep}"
    return rep
