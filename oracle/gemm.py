"""FP64 reference for dense, contiguous-grouped and masked-grouped FP8 GEMM.
TEST INFRASTRUCTURE ONLY.

Definition (DeepGEMM README, "Interfaces > Notices", page "Weight gradient
kernels for dense and MoE models #95"; same facts in the GeekNews digest,
section "GEMM interface और layout constraints"):

    D[m, n] = C[m, n] + sum_k  dec(A[m, k]) * sfa[k // 128][m]
                              * dec(B[n, k]) * sfb[n // 128][k // 128]

with A [M, K] and B [N, K] both K-contiguous ("NT": B is used transposed),
sfa stored transposed ([K/128][ld >= M]) and sfb stored [ceil(N/128)][K/128].
The kernel's per-128-K-slab promotion (partial products of one slab scaled
by sfa*sfb and added into FP32 accumulators, the MMA/promotion overlap the
Hacker News comments on the GeekNews page describe) is a regrouping of this
same sum, so the oracle is the plain dequantize-then-multiply definition.
In FP64 the dequantized operands are exact (4-bit x 24-bit significands),
so the only rounding is in the FP64 matmul itself.

Grouped variants (README sections "Grouped GEMMs (contiguous layout)" and
"Grouped GEMMs (masked layout)"):

* contiguous: rows of A are tokens of all experts concatenated; row r uses
  expert ``m_indices[r]``'s B; rows whose index is -1 (segment padding) are
  not outputs and must be left unwritten;
* masked: expert g owns A[g] with ``masked_m[g]`` valid leading rows (clamped
  to [0, M_max]); only those rows are outputs, the rest stay unwritten.

Every function returns FP64 values; pins live in ``tests/test_oracle_*.py``.
"""

from __future__ import annotations

import numpy as np

from .e4m3 import decode_e4m3

BLOCK = 128


def dequant_a(a: np.ndarray, sfa: np.ndarray, rows=None) -> np.ndarray:
    """A codes [M, K] with transposed scales sfa [K/128, ld] -> FP64 [len(rows), K].

    Element (m, k) is dec(A[m, k]) * sfa[k // 128][m].
    """
    m_all, k = a.shape
    rows = np.arange(m_all) if rows is None else np.asarray(rows)
    kb = k // BLOCK
    assert k % BLOCK == 0 and sfa.shape[0] == kb and sfa.shape[1] >= m_all
    vals = decode_e4m3(a[rows]).reshape(len(rows), kb, BLOCK)
    scale = sfa[:, rows].T.astype(np.float64)  # [rows, kb]
    return (vals * scale[:, :, None]).reshape(len(rows), k)


def dequant_b(b: np.ndarray, sfb: np.ndarray, cols=None) -> np.ndarray:
    """B codes [N, K] with block scales sfb [ceil(N/128), K/128] -> FP64 [len(cols), K].

    Element (n, k) is dec(B[n, k]) * sfb[n // 128][k // 128].
    """
    n_all, k = b.shape
    cols = np.arange(n_all) if cols is None else np.asarray(cols)
    kb = k // BLOCK
    assert sfb.shape == ((n_all + BLOCK - 1) // BLOCK, kb)
    vals = decode_e4m3(b[cols]).reshape(len(cols), kb, BLOCK)
    scale = sfb[cols // BLOCK].astype(np.float64)  # [cols, kb]
    return (vals * scale[:, :, None]).reshape(len(cols), k)


def ref_dense(a, sfa, b, sfb, c=None, rows=None, cols=None) -> np.ndarray:
    """FP64 D = C + A @ B.T, optionally only at the given rows x cols."""
    ad = dequant_a(a, sfa, rows)
    bd = dequant_b(b, sfb, cols)
    out = ad @ bd.T
    if c is not None:
        c = np.asarray(c, dtype=np.float64)
        if rows is not None:
            c = c[np.asarray(rows)]
        if cols is not None:
            c = c[:, np.asarray(cols)]
        out = out + c
    return out


def ref_contiguous(a, sfa, b, sfb, m_indices, rows=None, cols=None):
    """Contiguous M-grouped reference.

    a [M_total, K], sfa [K/128, ld >= M_total], b [G, N, K], sfb [G, NB, KB],
    m_indices int32 [M_total].  Returns ``(ref, written)``: ``ref`` FP64
    [len(rows), len(cols)] (NaN on rows that are not outputs) and ``written``
    bool [len(rows)].  A row is an output iff its index lies in [0, G).
    """
    m_total = a.shape[0]
    g_count, n = b.shape[0], b.shape[1]
    rows = np.arange(m_total) if rows is None else np.asarray(rows)
    cols = np.arange(n) if cols is None else np.asarray(cols)
    idx = np.asarray(m_indices)[rows]
    written = (idx >= 0) & (idx < g_count)
    out = np.full((len(rows), len(cols)), np.nan)
    for g in range(g_count):
        sel = np.nonzero(idx == g)[0]
        if len(sel) == 0:
            continue
        out[sel] = ref_dense(a, sfa, b[g], sfb[g], rows=rows[sel], cols=cols)
    return out, written


def ref_masked(a, sfa, b, sfb, masked_m, groups=None, cols=None):
    """Masked M-grouped reference.

    a [G, M_max, K], sfa [G, K/128, ld >= M_max], b [G, N, K], sfb [G, NB, KB],
    masked_m int32 [G].  Returns ``(ref, written)``: ``ref`` FP64
    [len(groups), M_max, len(cols)] (NaN beyond each group's valid rows) and
    ``written`` bool [len(groups), M_max].
    """
    g_count, m_max = a.shape[0], a.shape[1]
    n = b.shape[1]
    groups = np.arange(g_count) if groups is None else np.asarray(groups)
    cols = np.arange(n) if cols is None else np.asarray(cols)
    out = np.full((len(groups), m_max, len(cols)), np.nan)
    written = np.zeros((len(groups), m_max), dtype=bool)
    for i, g in enumerate(groups):
        mm = int(min(max(int(masked_m[g]), 0), m_max))
        if mm == 0:
            continue
        out[i, :mm] = ref_dense(a[g], sfa[g], b[g], sfb[g], rows=np.arange(mm), cols=cols)
        written[i, :mm] = True
    return out, written
