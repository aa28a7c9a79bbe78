"""UE8M0 (power-of-two) scale factors, packed four to a 32-bit word.
TEST INFRASTRUCTURE ONLY.

Source: DeepGEMM README, section "Interfaces > Notices" (page "Weight gradient
kernels for dense and MoE models #95"; the GeekNews digest "DeepGEMM: बारीक
scaling के जरिए साफ़ और efficient FP8 GEMM kernel" repeats it under "GEMM
interface और layout constraints"): one architecture takes FP32 scale factors,
the other takes UE8M0 scale factors with four of them packed into one 32-bit
integer.  The pages say no more, so these are the readings taken:

* UE8M0 is the OCP "E8M0" scale format: 8 exponent bits, bias 127, no sign,
  no mantissa.  Byte e means 2^(e - 127); byte 255 is NaN.
* The scale granularity is unchanged from the FP32 form: A has one scale per
  (row, 128-K block), B one per 128x128 block.
* Packing runs along K: byte j (j = 0 the least significant) of word q holds
  the scale of K block 4q + j.  A's words are stored MN-major like the FP32
  scales, ``sfa[q][m]`` with a leading dimension >= M; B's words are stored
  ``sfb[nb][q]``.  Bytes of the last word past the last K block are ignored.

With the scales decoded to FP64 the GEMM is exactly the FP32-scale
definition of ``gemm.py``, which this module calls.
"""

from __future__ import annotations

import math

import numpy as np

from .gemm import BLOCK, ref_contiguous, ref_dense, ref_masked


def ue8m0_closed_form(e: int) -> float:
    """Real value of one UE8M0 byte: 2^(e-127), NaN for 255."""
    e = int(e) & 0xFF
    if e == 0xFF:
        return math.nan
    return math.ldexp(1.0, e - 127)


UE8M0_TABLE = np.array([ue8m0_closed_form(e) for e in range(256)], dtype=np.float64)
UE8M0_TABLE.setflags(write=False)


def unpack_ue8m0(words: np.ndarray, kb: int, axis: int) -> np.ndarray:
    """Split 32-bit words into their four exponent bytes along ``axis``.

    ``words`` holds ceil(kb/4) words along ``axis``; the result holds kb uint8
    exponents there, byte j of word q landing at position 4q + j.
    """
    w = np.asarray(words)
    assert w.dtype in (np.int32, np.uint32)
    w = np.moveaxis(w.astype(np.int64) & 0xFFFFFFFF, axis, -1)
    assert w.shape[-1] == (kb + 3) // 4
    parts = [(w >> (8 * j)) & 0xFF for j in range(4)]
    e = np.stack(parts, axis=-1).reshape(*w.shape[:-1], 4 * w.shape[-1])[..., :kb]
    return np.moveaxis(e.astype(np.uint8), -1, axis)


def decode_ue8m0_sf(words: np.ndarray, kb: int, axis: int) -> np.ndarray:
    """Packed words -> FP64 scale factors (kb along ``axis``)."""
    return UE8M0_TABLE[unpack_ue8m0(words, kb, axis)]


def ref_dense_ue8m0(a, sfa_words, b, sfb_words, c=None, rows=None, cols=None):
    """FP64 D = C + A @ B.T with packed UE8M0 scales.

    sfa_words int32 [ceil(KB/4), ld >= M]; sfb_words int32 [ceil(N/128), ceil(KB/4)].
    """
    kb = a.shape[1] // BLOCK
    return ref_dense(a, decode_ue8m0_sf(sfa_words, kb, 0), b, decode_ue8m0_sf(sfb_words, kb, 1), c, rows, cols)


def ref_contiguous_ue8m0(a, sfa_words, b, sfb_words, m_indices, rows=None, cols=None):
    """Contiguous M-grouped reference with packed UE8M0 scales (sfb_words [G, NB, KQ])."""
    kb = a.shape[1] // BLOCK
    return ref_contiguous(a, decode_ue8m0_sf(sfa_words, kb, 0), b, decode_ue8m0_sf(sfb_words, kb, 2),
                          m_indices, rows, cols)


def ref_masked_ue8m0(a, sfa_words, b, sfb_words, masked_m, groups=None, cols=None):
    """Masked M-grouped reference with packed UE8M0 scales (sfa_words [G, KQ, ld])."""
    kb = a.shape[2] // BLOCK
    return ref_masked(a, decode_ue8m0_sf(sfa_words, kb, 1), b, decode_ue8m0_sf(sfb_words, kb, 2),
                      masked_m, groups, cols)


def ref_k_grouped_ue8m0(a, sfa_words, b, sfb_words, ks, c=None, groups=None, rows=None, cols=None):
    """K-grouped reference with packed UE8M0 scales, words along the global K blocks
    (sfa_words [ceil(KB/4), ld], sfb_words [NB, ceil(KB/4)])."""
    from .kgrouped import ref_k_grouped

    kb = a.shape[1] // BLOCK
    return ref_k_grouped(a, decode_ue8m0_sf(sfa_words, kb, 0), b, decode_ue8m0_sf(sfb_words, kb, 1), ks, c,
                         groups, rows, cols)
