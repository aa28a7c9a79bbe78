"""Scale-factor layout transform (oracle; test infrastructure only).

Source: DeepGEMM README as mirrored on "Weight gradient kernels for dense and
MoE models #95", section "Utilities" (transform the scaling factors into the
required layout; MN-major, TMA-aligned tensors, optionally packed into
UE8M0) and "Interfaces > Notices" (the LHS scale factor is transposed and
aligned; the UE8M0 form packs four per 32-bit int).

Input: per-row scales sf[g][r][kb] (row-major, one FP32 per row and 128-wide
K block).  Output, plainly:
  * FP32:  out[g][kb][r] = sf[g][r][kb], row stride ``ld`` >= r;
  * UE8M0: byte j of word out[g][q][r] is the biased exponent field of the
    FP32 sf[g][r][4q + j] (bits 30..23; exact for powers of two), 127 where
    4q + j >= KB.
Columns r >= rows are not part of the result (returned as NaN here so that a
comparison never reads them by accident).
"""

import numpy as np


def transform_sf(sf: np.ndarray, ld: int, ue8m0: bool = False) -> np.ndarray:
    """[R, KB] or [G, R, KB] FP32 -> [KB, ld] / [G, KB, ld] FP32 or int32 words."""
    x = np.asarray(sf, dtype=np.float32)
    squeeze = x.ndim == 2
    if squeeze:
        x = x[None]
    g, r, kb = x.shape
    assert ld >= r
    if not ue8m0:
        out = np.full((g, kb, ld), np.nan, dtype=np.float32)
        for gi in range(g):
            for k in range(kb):
                for row in range(r):
                    out[gi, k, row] = x[gi, row, k]
    else:
        kq = (kb + 3) // 4
        out = np.zeros((g, kq, ld), dtype=np.int64)
        bits = x.view(np.uint32)
        for gi in range(g):
            for q in range(kq):
                for row in range(r):
                    word = 0
                    for j in range(4):
                        k = 4 * q + j
                        byte = int((bits[gi, row, k] >> 23) & 0xFF) if k < kb else 127
                        word |= byte << (8 * j)
                    out[gi, q, row] = word
        out = out.astype(np.uint32).view(np.int32)
    return out[0] if squeeze else out
