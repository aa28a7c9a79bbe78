"""FP8 quantization of GEMM operands (the cast the GEMM's caller performs).
TEST INFRASTRUCTURE ONLY.

Sources: DeepGEMM README, section "Interfaces > Notices" (page "Weight
gradient kernels for dense and MoE models #95"): FP8 casting and
transposition are left to the caller, and the LHS scale factors must be in a
transposed, aligned layout; section "Utilities" lists helpers that put scale
factors into that layout (FP32, or packed UE8M0).  The page title of the
GeekNews digest "DeepGEMM: बारीक scaling के जरिए साफ़ और efficient FP8 GEMM
kernel" names the scheme: fine-grained scaling.  The pages give neither the
block shapes nor the scale rule, so the readings are:

* LHS / activations: one scale per (row, 128 consecutive K elements);
  RHS / weights: one scale per 128 x 128 block (the last row block may be
  partial);
* FP32 scales: s = amax / 448 evaluated in FP32 (448 is E4M3's largest
  finite magnitude), s = 1 for an all-zero block;
* UE8M0 scales: the smallest power of two s = 2^e with s >= fp32(amax / 448)
  (s = 1 for an all-zero block), stored as the byte e + 127;
* codes: y = x / s rounded to FP32, clamped to [-448, 448], then rounded to
  the nearest E4M3 value with ties to the even code; the sign of y is kept
  (negative values that round to zero give the code 0x80).

Where floating point decides the integer code, this module takes the same
FP32 steps the kernel takes (FP32 scale, FP32 quotient), then decides the
code exactly.  The E4M3 rounding below is written from the format's value
table (``e4m3.py``), not from any library cast.
"""

from __future__ import annotations

import numpy as np

from .e4m3 import E4M3_TABLE

BLOCK = 128
E4M3_MAX = 448.0

# Non-negative finite codes 0x00..0x7E have increasing values.
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALS = E4M3_TABLE[:0x7F]


def e4m3_encode_rne(y: np.ndarray) -> np.ndarray:
    """FP32 values with |y| <= 448 -> E4M3 codes, nearest value, ties to even code."""
    y = np.asarray(y, dtype=np.float32)
    mag = np.abs(y).astype(np.float64)
    assert np.isfinite(mag).all() and (mag <= E4M3_MAX).all()
    hi = np.searchsorted(_POS_VALS, mag, side="left")  # first value >= mag
    hi = np.minimum(hi, len(_POS_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _POS_VALS[lo]
    d_hi = _POS_VALS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_POS_CODES[hi] & 1) == 0))
    exact = _POS_VALS[hi] == mag
    code = np.where(exact | pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    return code | np.where(np.signbit(y), np.uint8(0x80), np.uint8(0))


def fp32_block_scale(amax: np.ndarray) -> np.ndarray:
    """s = fp32(amax / 448); 1 for amax == 0."""
    amax = np.asarray(amax, dtype=np.float32)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def ue8m0_block_exponent(amax: np.ndarray) -> np.ndarray:
    """Byte e + 127 of the smallest power of two 2^e >= fp32(amax / 448) (127 when amax == 0)."""
    t = (np.asarray(amax, dtype=np.float32) / np.float32(E4M3_MAX)).astype(np.float32)
    mant, ex = np.frexp(t.astype(np.float64))  # t = mant * 2^ex, mant in [0.5, 1)
    e = np.where(mant == 0.5, ex - 1, ex)
    e = np.where(t == 0, 0, e)
    return np.clip(e + 127, 0, 254).astype(np.uint8)


def _codes(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    y = (x.astype(np.float32) / s.astype(np.float32)).astype(np.float32)
    return e4m3_encode_rne(np.clip(y, -E4M3_MAX, E4M3_MAX))


def _pack_words(e: np.ndarray, axis: int) -> np.ndarray:
    """uint8 exponents along ``axis`` -> int32 words, 4 per word (byte j = block 4q + j), padding bytes 127."""
    e = np.moveaxis(np.asarray(e, dtype=np.int64), axis, -1)
    kb = e.shape[-1]
    kq = (kb + 3) // 4
    pad = np.full((*e.shape[:-1], 4 * kq), 127, dtype=np.int64)
    pad[..., :kb] = e
    pad = pad.reshape(*e.shape[:-1], kq, 4)
    w = pad[..., 0] | (pad[..., 1] << 8) | (pad[..., 2] << 16) | (pad[..., 3] << 24)
    return np.moveaxis(w.astype(np.uint32).view(np.int32), -1, axis)


def quant_per_token(x: np.ndarray, ld_sf: int | None = None, ue8m0: bool = False):
    """x [M, K] (FP32 or BF16 values) -> (codes uint8 [M, K], scales).

    Scales are stored transposed: FP32 [K/128, ld_sf] or UE8M0 words
    int32 [ceil(K/512), ld_sf]; ld_sf defaults to M rounded up to 4 and the
    padding columns are zero.
    """
    m, k = x.shape
    assert k % BLOCK == 0
    kb = k // BLOCK
    ld = (m + 3) // 4 * 4 if ld_sf is None else ld_sf
    xb = np.asarray(x, dtype=np.float32).reshape(m, kb, BLOCK)
    amax = np.abs(xb).max(axis=-1) if kb else np.zeros((m, 0), np.float32)
    if ue8m0:
        e = ue8m0_block_exponent(amax)  # [M, KB]
        s = np.ldexp(np.float32(1.0), e.astype(np.int32) - 127).astype(np.float32)
        sf = np.zeros(((kb + 3) // 4, ld), dtype=np.int32)
        sf[:, :m] = _pack_words(e, axis=1).T
    else:
        s = fp32_block_scale(amax)
        sf = np.zeros((kb, ld), dtype=np.float32)
        sf[:, :m] = s.T
    codes = _codes(xb, s[..., None]).reshape(m, k)
    return codes, sf


def quant_per_block(w: np.ndarray, ue8m0: bool = False):
    """w [N, K] -> (codes uint8 [N, K], scales FP32 [ceil(N/128), K/128] or UE8M0 words [ceil(N/128), ceil(K/512)])."""
    n, k = w.shape
    assert k % BLOCK == 0
    nb, kb = (n + BLOCK - 1) // BLOCK, k // BLOCK
    w32 = np.asarray(w, dtype=np.float32)
    codes = np.empty((n, k), dtype=np.uint8)
    e_all = np.empty((nb, kb), dtype=np.uint8)
    s_all = np.empty((nb, kb), dtype=np.float32)
    for i in range(nb):
        blk = w32[i * BLOCK:(i + 1) * BLOCK].reshape(-1, kb, BLOCK)
        amax = np.abs(blk).max(axis=(0, 2)) if kb else np.zeros(0, np.float32)
        if ue8m0:
            e_all[i] = ue8m0_block_exponent(amax)
            s = np.ldexp(np.float32(1.0), e_all[i].astype(np.int32) - 127).astype(np.float32)
        else:
            s = fp32_block_scale(amax)
        s_all[i] = s
        codes[i * BLOCK:(i + 1) * BLOCK] = _codes(blk, s[None, :, None]).reshape(-1, k)
    return codes, (_pack_words(e_all, axis=1) if ue8m0 else s_all)
