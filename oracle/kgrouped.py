"""K-grouped FP8 GEMM (MoE weight gradient).  TEST INFRASTRUCTURE ONLY.

Sources: DeepGEMM README, section "Grouped GEMMs (contiguous layout)" (page
"Weight gradient kernels for dense and MoE models #95"): besides the M-grouped
API there is a K-axis-grouped API for the MoE weight backward in which M and N
stay fixed.  The pull request text on the same page introduces FP8 x FP8 ->
FP32 weight-gradient GEMMs for dense and for MoE models.  The pages give no
signature, so the readings are:

* groups split the K axis: group g owns the K range
  [k_off[g], k_off[g] + ks[g]) with k_off the exclusive prefix sum of ks,
  every ks[g] a multiple of 128 (the contiguous-layout alignment), zero
  allowed;
* operands are K-contiguous ("NT", like the forward kernels; a caller holding
  token-major tensors transposes them first, which the README leaves to the
  caller): A [M, K_total], B [N, K_total];
* scales keep the forward scheme over the global K-block index:
  sfa[K_total/128][ld >= M] per (row, 128-K block), sfb[ceil(N/128)][K_total/128]
  per 128x128 block;
* each group has its own FP32 output: D[g] = C[g] + A[:, K_g] @ B[:, K_g].T,
  D and C of shape [G, M, N] (C may be D itself, which is the weight-gradient
  accumulation; C absent means zero).

This is the dense definition of ``gemm.py`` restricted to each group's K
range, and it is written that way.
"""

from __future__ import annotations

import numpy as np

from .gemm import BLOCK, ref_dense


def k_offsets(ks) -> np.ndarray:
    """Exclusive prefix sum of the group K sizes."""
    ks = np.asarray(ks, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(ks)[:-1]]) if len(ks) else np.zeros(0, np.int64)


def ref_k_grouped(a, sfa, b, sfb, ks, c=None, groups=None, rows=None, cols=None) -> np.ndarray:
    """FP64 [len(groups), len(rows), len(cols)] with D[g] = C[g] + A_g @ B_g.T."""
    ks = np.asarray(ks, dtype=np.int64)
    g_count = len(ks)
    m, n = a.shape[0], b.shape[0]
    assert (ks % BLOCK == 0).all() and (ks >= 0).all() and int(ks.sum()) == a.shape[1] == b.shape[1]
    groups = np.arange(g_count) if groups is None else np.asarray(groups)
    rows = np.arange(m) if rows is None else np.asarray(rows)
    cols = np.arange(n) if cols is None else np.asarray(cols)
    off = k_offsets(ks)
    out = np.zeros((len(groups), len(rows), len(cols)))
    for i, g in enumerate(groups):
        k0, kg = int(off[g]), int(ks[g])
        if kg > 0:
            kb0, kb1 = k0 // BLOCK, (k0 + kg) // BLOCK
            out[i] = ref_dense(a[:, k0:k0 + kg], sfa[kb0:kb1], b[:, k0:k0 + kg], sfb[:, kb0:kb1],
                               rows=rows, cols=cols)
        if c is not None:
            out[i] += np.asarray(c[g], dtype=np.float64)[np.ix_(rows, cols)]
    return out
