"""E4M3 decode table from the format's closed form.  TEST INFRASTRUCTURE ONLY.

The pages name the FP8 operand format only as E4M3 (DeepGEMM README, section
"V3.2 MQA kernels for the indexer", page "Weight gradient kernels for dense
and MoE models #95"; the GEMM inputs are FP8 per "Interfaces").  The reading
taken here is the OCP E4M3FN encoding: 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits, no infinities, NaN only where exponent and mantissa
bits are all ones, largest finite magnitude 448.

    exponent field e == 0  ->  (-1)^s * (m / 8) * 2^-6          (subnormal)
    otherwise              ->  (-1)^s * (1 + m / 8) * 2^(e - 7)
    e == 15 and m == 7     ->  NaN

Pinned in ``tests/test_oracle_e4m3.py`` against torch's independent
``float8_e4m3fn`` decode on all 256 codes and against spec values.
"""

import math

import numpy as np


def e4m3_closed_form(code: int) -> float:
    """Real value of one E4M3FN byte code (NaN for the two NaN codes)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_closed_form(c) for c in range(256)], dtype=np.float64)
E4M3_TABLE.setflags(write=False)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """uint8 codes of any shape -> FP64 values (exact)."""
    codes = np.asarray(codes)
    assert codes.dtype == np.uint8
    return E4M3_TABLE[codes]
