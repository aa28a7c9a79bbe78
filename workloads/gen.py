"""Seeded generators for the five synthetic workloads (and smaller variants).

Recipe (shared by the oracle and the HIP path, so quantization details never
affect parity):

* values are drawn from ``numpy.random.default_rng(seed)`` (PCG64) as FP32
  ``standard_normal``, in the order: group sizes, A, B, C;
* A is quantized per (row, 128-wide K block): ``s = amax / 448`` in FP32
  (``s = 1`` when the block is all zero), codes are ``E4M3(clamp(x/s))``
  with round-to-nearest-even (torch's CPU cast, OCP E4M3FN);
* B is quantized per 128x128 block with the same rule;
* A's scales are stored transposed (MN-major): ``sfa[kb][m]`` with a leading
  dimension rounded up to 4 floats (16 bytes) -- the transposed,
  aligned LHS scale layout the DeepGEMM README asks for ("Interfaces >
  Notices" on the page "Weight gradient kernels for dense and MoE models #95");
* B's scales are stored ``sfb[nb][kb]`` (``[g][nb][kb]`` when grouped).

The block size 128 and the amax/448 rule are this library's fixed reading of
"fine-grained scaling" (page title of the GeekNews digest "DeepGEMM: बारीक
scaling के जरिए साफ़ और efficient FP8 GEMM kernel"); the pages give no block size.
"""

from __future__ import annotations

import numpy as np
import torch

SF_BLOCK = 128
E4M3_MAX = 448.0
ALIGN_M = 128  # contiguous-layout segment alignment


def _cdiv(a: int, b: int) -> int:
    return (a + b - 1) // b


def sf_aligned_size(mn: int) -> int:
    """Leading dimension of a transposed FP32 scale tensor: ``mn`` rounded up to 4."""
    return _cdiv(mn, 4) * 4


def _to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """FP32 -> E4M3FN byte codes, RNE, after clamping to +-448.

    torch's cast maps out-of-range values to NaN instead of saturating, so the
    clamp comes first.
    """
    x = np.clip(x, -E4M3_MAX, E4M3_MAX).astype(np.float32, copy=False)
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _block_scale(amax: np.ndarray, pow2: bool = False) -> np.ndarray:
    """amax / 448 in FP32 (1 for an all-zero block); with ``pow2`` the next power of two up."""
    amax = amax.astype(np.float32, copy=False)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    if pow2:
        mant, ex = np.frexp(s.astype(np.float64))
        s = np.ldexp(1.0, np.where(mant == 0.5, ex - 1, ex)).astype(np.float32)
    s[amax == 0] = np.float32(1.0)
    return s


def quantize_per_row_block(x: np.ndarray, pow2: bool = False):
    """x: FP32 [R, K] -> (codes uint8 [R, K], scales FP32 [R, K/128])."""
    r, k = x.shape
    assert k % SF_BLOCK == 0
    xb = x.reshape(r, k // SF_BLOCK, SF_BLOCK)
    s = _block_scale(np.abs(xb).max(axis=-1), pow2)
    q = _to_e4m3_codes(xb / s[..., None])
    return q.reshape(r, k), s


def quantize_per_block(x: np.ndarray, pow2: bool = False):
    """x: FP32 [N, K] -> (codes uint8 [N, K], scales FP32 [ceil(N/128), K/128]).

    The last row block may be partial (N not a multiple of 128); its scale
    covers only the rows that exist.
    """
    n, k = x.shape
    assert k % SF_BLOCK == 0
    nb, kb = _cdiv(n, SF_BLOCK), k // SF_BLOCK
    codes = np.empty((n, k), dtype=np.uint8)
    s = np.empty((nb, kb), dtype=np.float32)
    for i in range(nb):
        blk = x[i * SF_BLOCK:(i + 1) * SF_BLOCK].reshape(-1, kb, SF_BLOCK)
        si = _block_scale(np.abs(blk).max(axis=(0, 2)), pow2)
        s[i] = si
        codes[i * SF_BLOCK:(i + 1) * SF_BLOCK] = _to_e4m3_codes(blk / si[None, :, None]).reshape(-1, k)
    return codes, s


def pack_ue8m0(scales: np.ndarray, axis: int) -> np.ndarray:
    """Power-of-two FP32 scales -> UE8M0 bytes (log2 + 127) packed four per int32
    along ``axis`` (byte j of word q = entry 4q + j; padding bytes 127)."""
    sc = np.moveaxis(np.asarray(scales, dtype=np.float64), axis, -1)
    mant, ex = np.frexp(sc)
    assert (mant == 0.5).all(), "UE8M0 scales must be powers of two"
    e = (ex - 1 + 127).astype(np.int64)
    assert ((e >= 0) & (e <= 254)).all()
    kb = e.shape[-1]
    kq = _cdiv(kb, 4)
    buf = np.full((*e.shape[:-1], 4 * kq), 127, dtype=np.uint8)
    buf[..., :kb] = e
    words = np.ascontiguousarray(buf).view("<u4").view(np.int32)
    moved = np.moveaxis(words, -1, axis)
    out = np.empty(moved.shape, dtype=np.int32)  # fresh array: canonical strides even for size-1 axes
    out[...] = moved
    return out


def sf_to_mn_major(sf_rows: np.ndarray, ld: int | None = None) -> np.ndarray:
    """[R, KB] per-row scales -> transposed [KB, ld] (zero-padded columns)."""
    r, kb = sf_rows.shape
    ld = sf_aligned_size(r) if ld is None else ld
    assert ld >= r and ld % 4 == 0
    out = np.zeros((kb, ld), dtype=np.float32)
    out[:, :r] = sf_rows.T
    return out


def _draw(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def _quantize_b(rng, n: int, k: int, pow2: bool = False):
    return quantize_per_block(_draw(rng, (n, k)), pow2)


def gen_dense(m: int, n: int, k: int, seed: int, with_c: bool = False,
              out_dtype: str = "bf16", ld_sfa: int | None = None, scale_fmt: str = "fp32"):
    """Dense D = C + A @ B.T inputs.

    Returns a dict: ``a`` uint8 [M,K], ``sfa`` FP32 [K/128, ld_sfa],
    ``b`` uint8 [N,K], ``sfb`` FP32 [ceil(N/128), K/128], ``c`` FP32 [M,N]
    or None (exactly representable in BF16 when ``out_dtype == 'bf16'``).
    With ``scale_fmt='ue8m0'`` the scales are powers of two and ``sfa`` /
    ``sfb`` are packed UE8M0 words: int32 [ceil(K/512), ld_sfa] and
    [ceil(N/128), ceil(K/512)].
    """
    ue = scale_fmt == "ue8m0"
    rng = np.random.default_rng(seed)
    a_codes, a_s = quantize_per_row_block(_draw(rng, (m, k)), ue)
    b_codes, b_s = _quantize_b(rng, n, k, ue)
    c = None
    if with_c:
        c = _draw(rng, (m, n))
        if out_dtype == "bf16":
            c = torch.from_numpy(c).to(torch.bfloat16).float().numpy()
    sfa = sf_to_mn_major(a_s, ld_sfa)
    if ue:
        sfa = pack_ue8m0(np.where(np.arange(sfa.shape[1]) < m, sfa, 1.0), axis=0)
        b_s = pack_ue8m0(b_s, axis=1)
    return dict(kind="dense", m=m, n=n, k=k, out_dtype=out_dtype, scale_fmt=scale_fmt,
                a=a_codes, sfa=sfa, b=b_codes, sfb=b_s, c=c)


def gen_contiguous(num_groups: int, n: int, k: int, seed: int, m_sizes=None,
                   m_low: int = 1, m_high: int = 8192, out_dtype: str = "bf16", scale_fmt: str = "fp32"):
    """M-grouped contiguous layout (MoE prefill / training forward).

    Group sizes are drawn uniform in [m_low, m_high] unless ``m_sizes`` is
    given; each expert segment is zero-padded to a multiple of 128 rows.
    ``m_indices`` (int32 [M_total]) holds the group id of each row and -1 on
    padding rows.
    """
    ue = scale_fmt == "ue8m0"
    rng = np.random.default_rng(seed)
    if m_sizes is None:
        m_sizes = rng.integers(m_low, m_high + 1, num_groups)
    m_sizes = np.asarray(m_sizes, dtype=np.int64)
    assert m_sizes.shape == (num_groups,) and (m_sizes >= 0).all()
    padded = [_cdiv(int(s), ALIGN_M) * ALIGN_M for s in m_sizes]
    m_total = int(sum(padded))
    real = int(m_sizes.sum())
    a_real_codes, a_real_s = quantize_per_row_block(_draw(rng, (real, k)), ue) if real else (
        np.zeros((0, k), np.uint8), np.zeros((0, k // SF_BLOCK), np.float32))
    a = np.zeros((m_total, k), dtype=np.uint8)
    a_s = np.ones((m_total, k // SF_BLOCK), dtype=np.float32)  # all-zero rows -> scale 1
    m_indices = np.full((m_total,), -1, dtype=np.int32)
    src = dst = 0
    for g, (s, p) in enumerate(zip(m_sizes, padded)):
        s = int(s)
        a[dst:dst + s] = a_real_codes[src:src + s]
        a_s[dst:dst + s] = a_real_s[src:src + s]
        m_indices[dst:dst + s] = g
        src += s
        dst += p
    nb, kb = _cdiv(n, SF_BLOCK), k // SF_BLOCK
    b = np.empty((num_groups, n, k), dtype=np.uint8)
    sfb = np.empty((num_groups, nb, kb), dtype=np.float32)
    for g in range(num_groups):  # drawing per group consumes the stream in the same order
        b[g], sfb[g] = _quantize_b(rng, n, k, ue)
    sfa = sf_to_mn_major(a_s)
    if ue:
        sfa = pack_ue8m0(np.where(np.arange(sfa.shape[1]) < m_total, sfa, 1.0), axis=0)
        sfb = pack_ue8m0(sfb, axis=2)
    return dict(kind="contiguous", m_total=m_total, n=n, k=k, num_groups=num_groups,
                out_dtype=out_dtype, scale_fmt=scale_fmt, m_sizes=m_sizes, a=a, sfa=sfa,
                b=b, sfb=sfb, m_indices=m_indices)


def gen_masked(num_groups: int, m_max: int, n: int, k: int, seed: int, masked_m=None,
               poison: bool = False, out_dtype: str = "bf16", scale_fmt: str = "fp32"):
    """M-grouped masked layout (MoE decode).

    ``masked_m[g]`` is drawn uniform in [0, m_max] unless given.  All
    ``m_max`` rows of every group are drawn; with ``poison=True`` the rows
    at or beyond ``masked_m[g]`` get NaN codes (0x7F) and NaN scales, which
    must not leak into valid rows.
    """
    ue = scale_fmt == "ue8m0"
    rng = np.random.default_rng(seed)
    if masked_m is None:
        masked_m = rng.integers(0, m_max + 1, num_groups)
    masked_m = np.asarray(masked_m, dtype=np.int32)
    assert masked_m.shape == (num_groups,)
    kb = k // SF_BLOCK
    ld = sf_aligned_size(m_max)
    a = np.empty((num_groups, m_max, k), dtype=np.uint8)
    sfa = np.ones((num_groups, kb, ld), dtype=np.float32)
    for g in range(num_groups):
        codes, s = quantize_per_row_block(_draw(rng, (m_max, k)), ue)
        a[g] = codes
        sfa[g, :, :m_max] = s.T
    nb = _cdiv(n, SF_BLOCK)
    b = np.empty((num_groups, n, k), dtype=np.uint8)
    sfb = np.empty((num_groups, nb, kb), dtype=np.float32)
    for g in range(num_groups):
        b[g], sfb[g] = _quantize_b(rng, n, k, ue)
    if ue:
        sfa = pack_ue8m0(sfa, axis=1)
        sfb = pack_ue8m0(sfb, axis=2)
    if poison:
        for g in range(num_groups):
            mm = int(np.clip(masked_m[g], 0, m_max))
            a[g, mm:] = 0x7F
            if ue:
                sfa[g, :, mm:m_max] = -1  # every byte 255: NaN scales
            else:
                sfa[g, :, mm:m_max] = np.float32(np.nan)
    return dict(kind="masked", num_groups=num_groups, m_max=m_max, n=n, k=k, scale_fmt=scale_fmt,
                out_dtype=out_dtype, masked_m=masked_m, a=a, sfa=sfa, b=b, sfb=sfb)


def gen_k_grouped(num_groups: int, m: int, n: int, seed: int, ks=None, k_low: int = 1,
                  k_high: int = 8192, with_c: bool = True, scale_fmt: str = "fp32"):
    """K-grouped weight-gradient inputs: groups split K (tokens of each expert).

    Group token counts are drawn uniform in [k_low, k_high] unless ``ks`` is
    given, then padded up to multiples of 128 (the contiguous-layout
    alignment); draw order: counts, A, B, C.  A [M, K_total] is quantized per
    (row, 128-K block), B [N, K_total] per 128x128 block, C FP32 [G, M, N].
    With ``scale_fmt='ue8m0'`` the scales are powers of two packed as UE8M0
    words along the global K blocks (as for the dense GEMM).
    """
    ue = scale_fmt == "ue8m0"
    rng = np.random.default_rng(seed)
    if ks is None:
        ks = rng.integers(k_low, k_high + 1, num_groups)
        ks = np.array([_cdiv(int(v), ALIGN_M) * ALIGN_M for v in ks], dtype=np.int32)
    ks = np.asarray(ks, dtype=np.int32)
    assert ks.shape == (num_groups,) and (ks % SF_BLOCK == 0).all() and (ks >= 0).all()
    k_total = int(ks.sum())
    a_codes, a_s = quantize_per_row_block(_draw(rng, (m, k_total)), ue)
    b_codes, b_s = _quantize_b(rng, n, k_total, ue)
    c = _draw(rng, (num_groups, m, n)) if with_c else None
    sfa = sf_to_mn_major(a_s)
    if ue:
        sfa = pack_ue8m0(np.where(np.arange(sfa.shape[1]) < m, sfa, 1.0), axis=0)
        b_s = pack_ue8m0(b_s, axis=1)
    return dict(kind="k_grouped", num_groups=num_groups, m=m, n=n, k=k_total, ks=ks, scale_fmt=scale_fmt,
                a=a_codes, sfa=sfa, b=b_codes, sfb=b_s, c=c)


def gen_quant_input(rows: int, k: int, seed: int, dtype: str = "bf16"):
    """Raw activations / weights for the FP8 cast: N(0,1) rows with a per-row
    magnitude spread of e^U(-4, 4), one all-zero 128-block in the first row
    (when K >= 256) and a few large outliers; returned as FP32 values that are
    exact in ``dtype`` ('bf16' or 'fp32')."""
    rng = np.random.default_rng(seed)
    x = _draw(rng, (rows, k)) * np.exp(rng.uniform(-4, 4, (rows, 1))).astype(np.float32)
    if rows and k >= 256:
        x[0, 128:256] = 0
    if rows * k:
        idx = rng.integers(0, rows * k, max(1, rows * k // 100000))
        x.reshape(-1)[idx] *= np.float32(50.0)
    if dtype == "bf16":
        x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    return x


def gen_mqa(s: int, s_kv: int, h: int, d: int, seed: int, ranges: str = "causal"):
    """Inputs of the MQA-logits kernel.

    q: E4M3 codes [S, H, D] of N(0,1) values (q carries no scale); kv: E4M3
    codes [S_kv, D] of N(0,1) rows quantized per row with sf = amax / 448;
    weights FP32 [S, H] ~ N(0,1)/sqrt(H); draw order q, kv, weights, ranges.
    ``ranges='causal'``: query i of the last S positions sees keys
    [0, S_kv - S + i + 1) (prefill with a cached prefix); ``'random'``:
    windows with random starts and lengths in [0, S_kv], some empty, some
    running past S_kv, some starting below 0.
    """
    rng = np.random.default_rng(seed)
    q = _to_e4m3_codes(_draw(rng, (s, h, d)))
    kv_x = _draw(rng, (s_kv, d))
    amax = np.abs(kv_x).max(axis=1)
    sf = _block_scale(amax)
    kv = _to_e4m3_codes(kv_x / sf[:, None])
    w = (_draw(rng, (s, h)) / np.float32(np.sqrt(h))).astype(np.float32)
    if ranges == "causal":
        ke = (s_kv - s + np.arange(s) + 1).astype(np.int32)
        ks = np.zeros(s, np.int32)
    else:
        ks = rng.integers(-8, s_kv, s).astype(np.int32)
        ke = (ks + rng.integers(0, s_kv // 2 + 2, s)).astype(np.int32)
        if s >= 2:
            ke[1] = ks[1]  # an empty range
    return dict(kind="mqa", s=s, s_kv=s_kv, h=h, d=d, q=q, kv=kv, sf=sf, w=w, ks=ks, ke=ke)


# (N, K) pairs and M values of the dense sweep; case i = m_index * 5 + nk_index, seed 100 + i.
DENSE_SWEEP_NK = [(2112, 7168), (24576, 1536), (7168, 16384), (4096, 7168), (7168, 2048)]
DENSE_SWEEP_M = [64, 128, 4096]
DENSE_SWEEP = [(m, n, k) for m in DENSE_SWEEP_M for (n, k) in DENSE_SWEEP_NK]

WORKLOAD_NAMES = ("baseline", "dense_small", "dense_sweep", "contiguous_moe", "masked_decode", "dense_long_k_acc",
                  "dense_sweep_ue8m0", "contiguous_moe_ue8m0", "masked_decode_ue8m0", "k_grouped_wgrad",
                  "quant_moe", "mqa_logits")


def workload(name: str):
    """Case descriptors (no data) for the named workload.

    Each descriptor is a dict with a ``gen`` callable producing the inputs.
    """
    if name == "baseline":
        # the five benchmark configurations in order: small dense, the dense sweep,
        # contiguous MoE, masked decode (both shapes), long-K dense with FP32 C/D
        out = []
        for cfg, part in ((0, "dense_small"), (1, "dense_sweep"), (2, "contiguous_moe"), (3, "masked_decode"),
                          (4, "dense_long_k_acc")):
            for d in workload(part):
                out.append(dict(d, config=cfg))
        return out
    if name == "dense_small":
        return [dict(label="dense M=128 N=256 K=512", kind="dense", m=128, n=256, k=512,
                     gen=lambda: gen_dense(128, 256, 512, seed=0))]
    if name == "dense_sweep":
        out = []
        for i, (m, n, k) in enumerate(DENSE_SWEEP):
            out.append(dict(label=f"dense M={m} N={n} K={k}", kind="dense", m=m, n=n, k=k,
                            gen=(lambda m=m, n=n, k=k, i=i: gen_dense(m, n, k, seed=100 + i))))
        return out
    if name == "contiguous_moe":
        return [dict(label="contiguous G=8 N=4096 K=7168", kind="contiguous", n=4096, k=7168,
                     num_groups=8, gen=lambda: gen_contiguous(8, 4096, 7168, seed=2))]
    if name == "masked_decode":
        out = []
        for j, (n, k) in enumerate([(4096, 7168), (7168, 2048)]):
            out.append(dict(label=f"masked G=16 Mmax=256 N={n} K={k}", kind="masked", n=n, k=k,
                            num_groups=16, m_max=256,
                            gen=(lambda n=n, k=k, j=j: gen_masked(16, 256, n, k, seed=30 + j))))
        return out
    if name == "dense_sweep_ue8m0":
        out = []
        for i, (m, n, k) in enumerate(DENSE_SWEEP):
            out.append(dict(label=f"dense ue8m0 M={m} N={n} K={k}", kind="dense", m=m, n=n, k=k,
                            gen=(lambda m=m, n=n, k=k, i=i: gen_dense(m, n, k, seed=100 + i, scale_fmt="ue8m0"))))
        return out
    if name == "contiguous_moe_ue8m0":
        return [dict(label="contiguous ue8m0 G=8 N=4096 K=7168", kind="contiguous", n=4096, k=7168, num_groups=8,
                     gen=lambda: gen_contiguous(8, 4096, 7168, seed=2, scale_fmt="ue8m0"))]
    if name == "masked_decode_ue8m0":
        out = []
        for j, (n, k) in enumerate([(4096, 7168), (7168, 2048)]):
            out.append(dict(label=f"masked ue8m0 G=16 Mmax=256 N={n} K={k}", kind="masked", n=n, k=k,
                            num_groups=16, m_max=256,
                            gen=(lambda n=n, k=k, j=j: gen_masked(16, 256, n, k, seed=30 + j, scale_fmt="ue8m0"))))
        return out
    if name == "k_grouped_wgrad":
        # weight gradient of the contiguous MoE layer: dW[g] [4096, 7168] over each expert's tokens
        return [dict(label="k-grouped wgrad G=8 M=4096 N=7168 K_g~U[1,8192]", kind="k_grouped", m=4096, n=7168,
                     num_groups=8, gen=lambda: gen_k_grouped(8, 4096, 7168, seed=5))]
    if name == "k_grouped_wgrad_ue8m0":
        return [dict(label="k-grouped wgrad ue8m0 G=8 M=4096 N=7168 K_g~U[1,8192]", kind="k_grouped", m=4096,
                     n=7168, num_groups=8, gen=lambda: gen_k_grouped(8, 4096, 7168, seed=5, scale_fmt="ue8m0"))]
    if name == "quant_moe":
        # the casts feeding the contiguous MoE GEMM: token activations (1x128
        # scales, transposed) and the 8 experts' weights (128x128 scales), BF16 in
        return [dict(label="per-token cast BF16 [33280, 7168]", kind="quant_token", m=33280, k=7168,
                     gen=lambda: dict(kind="quant_token", m=33280, k=7168, dtype="bf16",
                                      x=gen_quant_input(33280, 7168, seed=6))),
                dict(label="per-block cast BF16 [32768, 7168]", kind="quant_block", m=32768, k=7168,
                     gen=lambda: dict(kind="quant_block", m=32768, k=7168, dtype="bf16",
                                      x=gen_quant_input(32768, 7168, seed=7)))]
    if name == "mqa_logits":
        # indexer prefill: 4096 new tokens over a 4096-token cached prefix, 64 heads of dim 128
        return [dict(label="mqa logits S=4096 S_kv=8192 H=64 D=128 causal", kind="mqa", s=4096, s_kv=8192,
                     gen=lambda: gen_mqa(4096, 8192, 64, 128, seed=8, ranges="causal"))]
    if name == "dense_long_k_acc":
        return [dict(label="dense+C M=8192 N=8192 K=16384 fp32", kind="dense", m=8192, n=8192, k=16384,
                     gen=lambda: gen_dense(8192, 8192, 16384, seed=4, with_c=True, out_dtype="fp32"))]
    raise KeyError(name)
