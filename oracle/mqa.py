"""Weighted-ReLU MQA logits (the lightning-indexer scoring kernel).
TEST INFRASTRUCTURE ONLY.

Source: DeepGEMM README, section "V3.2 MQA kernels for the indexer" (page
"Weight gradient kernels for dense and MoE models #95"; the GeekNews digest
"DeepGEMM: बारीक scaling के जरिए साफ़ और efficient FP8 GEMM kernel" lists the
same inputs under its MQA section).  The non-paged form takes

* q: E4M3 [S, H, D] (no scale factor),
* kv: E4M3 [S_kv, D] with one FP32 scale per kv row, sf [S_kv],
* weights: FP32 [S, H],
* per-query K ranges [ks[i], ke[i]) (int32 [S] each),
* clean_logits: whether the positions outside the range become -inf,

and returns logits [S, S_kv] with, for j in the range of query i,

    out[i, j] = sum_h  w[i, h] * relu( sum_d dec(q[i, h, d]) * dec(kv[j, d]) * sf[j] ).

Readings where the pages are silent: the output is FP32; ks and ke are
clamped to [0, S_kv] and an empty range writes no logit; without
clean_logits the positions outside the range are left untouched (the caller's
buffer keeps its contents); with it they are set to -inf.
"""

from __future__ import annotations

import numpy as np

from .e4m3 import decode_e4m3


def ref_mqa_logits(q, kv, kv_sf, weights, ks, ke, clean_logits: bool, rows=None):
    """FP64 [len(rows), S_kv]; NaN marks positions the kernel must leave untouched."""
    s, h, d = q.shape
    s_kv = kv.shape[0]
    rows = np.arange(s) if rows is None else np.asarray(rows)
    kvd = decode_e4m3(kv) * np.asarray(kv_sf, dtype=np.float64)[:, None]  # [S_kv, D]
    out = np.full((len(rows), s_kv), -np.inf if clean_logits else np.nan)
    w = np.asarray(weights, dtype=np.float64)
    for r, i in enumerate(rows):
        lo = min(max(int(ks[i]), 0), s_kv)
        hi = min(max(int(ke[i]), 0), s_kv)
        if hi <= lo:
            continue
        qi = decode_e4m3(q[i])  # [H, D]
        logits = qi @ kvd[lo:hi].T  # [H, hi - lo]
        out[r, lo:hi] = (np.maximum(logits, 0.0) * w[i][:, None]).sum(axis=0)
    return out
