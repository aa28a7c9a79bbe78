"""Pins for the oracle's E4M3 decode table (CPU only).

The table is built from the format's closed form; here it is checked against
an independent decoder (torch's ``float8_e4m3fn`` view), against values fixed
by the OCP E4M3 definition (tests/golden/e4m3_ocp_spec_values.txt), and
against structural invariants (monotonic, sign-symmetric, 253 distinct
finite values).
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import E4M3_TABLE, decode_e4m3, e4m3_closed_form

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_spec_values.txt")


def test_table_matches_torch_decoder_on_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = E4M3_TABLE
    nan_lib, nan_ours = np.isnan(lib), np.isnan(ours)
    assert (nan_lib == nan_ours).all()
    assert np.array_equal(lib[~nan_lib], ours[~nan_ours])
    # signed zero is kept
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_nan_codes_and_no_infinity():
    nan_codes = [c for c in range(256) if math.isnan(E4M3_TABLE[c])]
    assert nan_codes == [0x7F, 0xFF]
    assert not np.isinf(E4M3_TABLE).any()
    assert np.nanmax(np.abs(E4M3_TABLE)) == 448.0


def test_golden_spec_values():
    with open(GOLDEN) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 10
    for code_s, val_s in rows:
        code = int(code_s, 16)
        want = float(val_s)
        got = E4M3_TABLE[code]
        if math.isnan(want):
            assert math.isnan(got), code_s
        else:
            assert got == want, (code_s, got, want)
            assert math.copysign(1.0, got) == math.copysign(1.0, want), code_s


def test_monotonic_and_sign_symmetric():
    pos = E4M3_TABLE[0x00:0x7F]
    assert (np.diff(pos) > 0).all()
    for c in range(0x80):
        a, b = E4M3_TABLE[c], E4M3_TABLE[c ^ 0x80]
        if math.isnan(a):
            assert math.isnan(b)
        else:
            assert a == -b


def test_distinct_finite_values():
    fin = E4M3_TABLE[np.isfinite(E4M3_TABLE)]
    assert len(set(fin.tolist())) == 253  # +0 and -0 compare equal


def test_closed_form_subnormal_spacing():
    # subnormals are evenly spaced by 2^-9 and meet the first normal at 2^-6
    sub = [e4m3_closed_form(c) for c in range(0, 8)]
    assert sub == [i * 2.0 ** -9 for i in range(8)]
    assert e4m3_closed_form(8) == 2.0 ** -6


def test_decode_shape_and_dtype():
    codes = np.arange(256, dtype=np.uint8).reshape(16, 16)
    out = decode_e4m3(codes)
    assert out.dtype == np.float64 and out.shape == (16, 16)
    with pytest.raises(AssertionError):
        decode_e4m3(codes.astype(np.int32))
