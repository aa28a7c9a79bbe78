"""Python binding of libdg (fine-grained-scaled FP8 GEMM for MI355X / gfx950).

A thin ctypes layer over the C ABI in ``include/dg.h``: it checks tensor
dtypes/devices, passes ``data_ptr()`` values and the current HIP stream, and
raises ``RuntimeError`` with the library's status text on failure.  All
arithmetic runs in the HIP kernels; PyTorch only provides device memory and
the stream.  Names mirror the DeepGEMM README ("Interfaces", "Utilities")
as mirrored on the page "Weight gradient kernels for dense and MoE models #95":

* ``fp8_gemm_nt((a, sfa), (b, sfb), d, c=None, workspace=None)``
* ``m_grouped_fp8_gemm_nt_contiguous((a, sfa), (b, sfb), d, m_indices)``
* ``m_grouped_fp8_gemm_nt_masked((a, sfa), (b, sfb), d, masked_m, expected_m)``
* ``k_grouped_fp8_gemm_nt_contiguous((a, sfa), (b, sfb), d, ks, c=None)``
* ``wgrad_fp8_gemm_nt((a, sfa), (b, sfb), d)`` and
  ``k_grouped_wgrad_fp8_gemm_nt((a, sfa), (b, sfb), d, ks)`` (D += ..., FP32)
* ``per_token_cast_to_fp8(x, q, sf)`` and ``per_block_cast_to_fp8(w, q, sf)``
  (the caller's FP8 cast, writing the scale layouts the GEMMs take)
* ``fp8_mqa_logits(q, (kv, kv_sf), weights, ks, ke, clean_logits, out)``
  (README "V3.2 MQA kernels for the indexer")
* ``get_mk_alignment_for_contiguous_layout()``, ``get_sf_aligned_size(mn)``,
  ``set_num_cus(n)`` / ``get_num_cus()``, ``get_workspace_size(m, n, k)`` and
  ``alloc_workspace(m, n, k)``

Skinny dense GEMMs (M <= 128) split K across workgroups and need a split-K
workspace (``get_workspace_size``): zero-filled device memory that the caller
keeps and passes to every call (``alloc_workspace`` makes one); each call
leaves it ready for the next.  Without one, the dense calls take a fresh
workspace from torch's allocator per call and clear its counters (one small
fill kernel before the GEMM).

The three M-side GEMMs take either FP32 scales or UE8M0 scales packed four
per int32 along K (the README's "Interfaces > Notices" names both formats);
the binding picks the entry point from the scale tensors' dtype.

Operands follow the ``(tensor, scale)`` pair convention of the README:
``a`` is E4M3 (``torch.float8_e4m3fn`` or ``torch.uint8`` codes) ``[M, K]``
(masked: ``[G, M_max, K]``), ``sfa`` is FP32 ``[K/128, ld]`` transposed
(masked: ``[G, K/128, ld]``), ``b`` is E4M3 ``[N, K]`` (grouped
``[G, N, K]``), ``sfb`` is FP32 ``[ceil(N/128), K/128]`` (grouped
``[G, ceil(N/128), K/128]``), ``d`` is a caller-allocated BF16 or FP32 tensor.
With UE8M0 scales, ``sfa`` is int32 ``[ceil(K/512), ld]`` (masked
``[G, ceil(K/512), ld]``) and ``sfb`` int32 ``[ceil(N/128), ceil(K/512)]``
(grouped ``[G, ...]``).
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "fp8_gemm_nt",
    "m_grouped_fp8_gemm_nt_contiguous",
    "m_grouped_fp8_gemm_nt_masked",
    "k_grouped_fp8_gemm_nt_contiguous",
    "wgrad_fp8_gemm_nt",
    "k_grouped_wgrad_fp8_gemm_nt",
    "per_token_cast_to_fp8",
    "per_block_cast_to_fp8",
    "fp8_mqa_logits",
    "transform_sf_into_required_layout",
    "get_mn_major_tma_aligned_tensor",
    "get_mn_major_tma_aligned_packed_ue8m0_tensor",
    "get_mk_alignment_for_contiguous_layout",
    "get_sf_aligned_size",
    "set_num_cus",
    "get_num_cus",
    "get_workspace_size",
    "alloc_workspace",
    "set_num_sms",
    "get_num_sms",
    "get_tma_aligned_size",
    "library_path",
    "load_library",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdg.so")
_lib = None

_DTYPES = {torch.bfloat16: 0, torch.float32: 1}
_STATUS = {0: "DG_SUCCESS"}

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int
_sz = ctypes.c_size_t

_SIGNATURES = {
    "dg_fp8_gemm_nt": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _i64, _i32,
                              _i32, _i32, _i32, _vp, _sz, _vp]),
    "dg_get_workspace_size": (_sz, [_i32, _i32, _i32]),
    "dg_fp8_gemm_nt_noalloc": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _i64, _i32,
                                      _i32, _i32, _i32, _vp]),
    "dg_m_grouped_fp8_gemm_nt_contiguous": (_i32, [_vp, _vp, _i64, _vp, _vp, _vp, _i32, _vp,
                                                   _i32, _i32, _i32, _i32, _vp]),
    "dg_m_grouped_fp8_gemm_nt_masked": (_i32, [_vp, _vp, _i64, _vp, _vp, _vp, _i32, _vp,
                                               _i32, _i32, _i32, _i32, _i32, _vp]),
    "dg_fp8_gemm_nt_ue8m0": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _i64, _i32,
                                    _i32, _i32, _i32, _vp, _sz, _vp]),
    "dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0": (_i32, [_vp, _vp, _i64, _vp, _vp, _vp, _i32, _vp,
                                                         _i32, _i32, _i32, _i32, _vp]),
    "dg_m_grouped_fp8_gemm_nt_masked_ue8m0": (_i32, [_vp, _vp, _i64, _vp, _vp, _vp, _i32, _vp,
                                                     _i32, _i32, _i32, _i32, _i32, _vp]),
    "dg_k_grouped_fp8_gemm_nt_contiguous": (_i32, [_vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp,
                                                   _i32, _i32, _i32, _i32, _vp]),
    "dg_wgrad_fp8_gemm_nt": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _i64, _i32, _i32, _i32, _vp, _sz,
                                    _vp]),
    "dg_k_grouped_wgrad_fp8_gemm_nt": (_i32, [_vp, _vp, _i64, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]),
    "dg_k_grouped_fp8_gemm_nt_contiguous_ue8m0": (_i32, [_vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp,
                                                         _i32, _i32, _i32, _i32, _vp]),
    "dg_k_grouped_wgrad_fp8_gemm_nt_ue8m0": (_i32, [_vp, _vp, _i64, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                                    _vp]),
    "dg_per_token_cast_to_fp8": (_i32, [_vp, _i64, _i32, _vp, _i64, _vp, _i64, _i32, _i32, _i32, _vp]),
    "dg_per_block_cast_to_fp8": (_i32, [_vp, _i64, _i32, _vp, _i64, _vp, _i32, _i32, _i32, _vp]),
    "dg_fp8_mqa_logits": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp]),
    "dg_transform_sf_into_required_layout": (_i32, [_vp, _vp, _i32, _i32, _i32, _i64, _i32, _vp]),
    "dg_get_mk_alignment_for_contiguous_layout": (_i32, []),
    "dg_get_sf_aligned_size": (_i64, [_i64]),
    "dg_set_num_cus": (_i32, [_i32]),
    "dg_get_num_cus": (_i32, []),
    "dg_internal_set_tile_n": (_i32, [_i32]),
    "dg_internal_dense_plan": (_i32, [_i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "dg_status_string": (ctypes.c_char_p, [_i32]),
    "dg_last_hip_error": (ctypes.c_char_p, []),
}


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libdg.so (built in-tree by ``build.py``); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libdg.so not built: run `python -m moe_grouped_gemm_tiles_amd.build` "
                          f"(expected at {_LIB_PATH})")
    lib = ctypes.CDLL(_LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = load_library()
        msg = lib.dg_status_string(status).decode()
        hip = lib.dg_last_hip_error().decode()
        raise RuntimeError(msg + (f" ({hip})" if hip and status == 3 else ""))


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _unit_last_stride(t: torch.Tensor) -> bool:
    return t.numel() == 0 or t.size(-1) == 1 or t.stride(-1) == 1


def _ld(t: torch.Tensor, dim: int = 0, align: int = 1) -> int:
    """Leading dimension (elements between consecutive indices of ``dim``).

    A dimension of size 1 may carry any stride in torch (and numpy), so there
    the dense row length, rounded up to ``align`` elements, is passed instead;
    the library never steps along that dimension then.
    """
    if t.size(dim) > 1:
        return t.stride(dim)
    row = 1
    for s in t.shape[dim + 1:]:
        row *= s
    return (row + align - 1) // align * align


def _fp8(t: torch.Tensor, name: str):
    if t.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise TypeError(f"{name} must be torch.float8_e4m3fn or uint8 codes, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not _unit_last_stride(t):
        raise ValueError(f"{name} must be K-contiguous")


def _f32(t: torch.Tensor, name: str):
    if t.dtype != torch.float32 or not t.is_cuda:
        raise TypeError(f"{name} must be a float32 GPU tensor")
    if not _unit_last_stride(t):
        raise ValueError(f"{name} must be contiguous in its last dimension")


def _sf(sfa: torch.Tensor, sfb: torch.Tensor) -> bool:
    """Checks a scale pair; True for packed UE8M0 (int32), False for FP32."""
    if sfa.dtype != sfb.dtype or sfa.dtype not in (torch.float32, torch.int32):
        raise TypeError("sfa and sfb must both be float32 (FP32 scales) or both int32 (packed UE8M0)")
    for t, nm in ((sfa, "sfa"), (sfb, "sfb")):
        if not t.is_cuda:
            raise TypeError(f"{nm} must be a GPU tensor")
        if not _unit_last_stride(t):
            raise ValueError(f"{nm} must be contiguous in its last dimension")
    return sfa.dtype == torch.int32


def _sf_rows(k: int, ue8m0: bool) -> int:
    """Scale rows along K: K/128 FP32 scales, or ceil(K/512) packed UE8M0 words."""
    return (k // 128 + 3) // 4 if ue8m0 else k // 128


def _out(t: torch.Tensor, name: str = "d") -> int:
    if t.dtype not in _DTYPES or not t.is_cuda:
        raise TypeError(f"{name} must be a bfloat16 or float32 GPU tensor")
    if not _unit_last_stride(t):
        raise ValueError(f"{name} must be contiguous in its last dimension")
    return _DTYPES[t.dtype]


def _dense_contig(t: torch.Tensor, name: str):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def get_workspace_size(m: int, n: int, k: int) -> int:
    """Bytes of split-K workspace a dense M x N x K call needs on the current device (0: none)."""
    return int(load_library().dg_get_workspace_size(m, n, k))


def alloc_workspace(m: int, n: int, k: int, device=None) -> torch.Tensor | None:
    """A zero-filled split-K workspace for dense M x N x K calls (None when they need none).
    Keep it and pass it to every call of that shape; calls sharing it must not overlap."""
    size = get_workspace_size(m, n, k)
    if size == 0:
        return None
    return torch.zeros(size, dtype=torch.uint8, device=device if device is not None else torch.cuda.current_device())


_WS_ALIGN = 256  # the library's alignment rule for workspaces


def _workspace(m: int, n: int, k: int, workspace: torch.Tensor | None, like: torch.Tensor):
    """(pointer, bytes) of the split-K workspace for a dense call; without one, a fresh
    zero-filled workspace from torch's allocator (filled on the current stream)."""
    size = get_workspace_size(m, n, k)
    if size == 0:
        return None, 0
    if workspace is None:
        workspace = torch.zeros(size + _WS_ALIGN, dtype=torch.uint8, device=like.device)
        off = (-workspace.data_ptr()) % _WS_ALIGN
        workspace = workspace[off:off + size]
    elif not workspace.is_cuda or workspace.device != like.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the output's device")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def fp8_gemm_nt(a_pair, b_pair, d: torch.Tensor, c: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None):
    """D = C + A @ B.T with A [M,K], B [N,K] E4M3 and FP32 or packed-UE8M0 fine-grained scales.
    ``workspace``: split-K workspace for skinny M (``alloc_workspace``), or None."""
    lib = load_library()
    a, sfa = a_pair
    b, sfb = b_pair
    _fp8(a, "a")
    _fp8(b, "b")
    ue = _sf(sfa, sfb)
    _dense_contig(sfb, "sfb")
    dt = _out(d)
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k or d.shape != (m, n):
        raise ValueError(f"shape mismatch: a {tuple(a.shape)}, b {tuple(b.shape)}, d {tuple(d.shape)}")
    kr = _sf_rows(k, ue)
    if sfa.dim() != 2 or sfa.shape[0] != kr or sfb.shape != ((n + 127) // 128, kr):
        raise ValueError(f"scale shapes: sfa {tuple(sfa.shape)}, sfb {tuple(sfb.shape)}")
    c_ptr, ldc = None, 0
    if c is not None:
        if c.dtype != d.dtype or c.shape != d.shape or not _unit_last_stride(c) or not c.is_cuda:
            raise ValueError("c must match d's dtype and shape")
        c_ptr, ldc = c.data_ptr(), _ld(c, 0, 16 // c.element_size())
    fn = lib.dg_fp8_gemm_nt_ue8m0 if ue else lib.dg_fp8_gemm_nt
    es = d.element_size()
    ws, ws_bytes = _workspace(m, n, k, workspace, d)
    st = fn(a.data_ptr(), _ld(a, 0, 16), sfa.data_ptr(), _ld(sfa, 0, 4), b.data_ptr(), _ld(b, 0, 16),
            sfb.data_ptr(), c_ptr, ldc, d.data_ptr(), _ld(d, 0, 16 // es), dt, m, n, k, ws, ws_bytes, _stream(d))
    _check(st)
    return d


def m_grouped_fp8_gemm_nt_contiguous(a_pair, b_pair, d: torch.Tensor, m_indices: torch.Tensor):
    """Contiguous-layout M-grouped GEMM; rows whose group index is -1 are left unwritten."""
    lib = load_library()
    a, sfa = a_pair
    b, sfb = b_pair
    for t, nm in ((a, "a"), (b, "b"), (sfb, "sfb"), (d, "d"), (m_indices, "m_indices")):
        _dense_contig(t, nm)
    _fp8(a, "a")
    _fp8(b, "b")
    ue = _sf(sfa, sfb)
    dt = _out(d)
    if m_indices.dtype != torch.int32 or not m_indices.is_cuda:
        raise TypeError("m_indices must be an int32 GPU tensor")
    m_total, k = a.shape
    g, n, kb_ = b.shape
    if kb_ != k or d.shape != (m_total, n) or m_indices.shape != (m_total,):
        raise ValueError("shape mismatch")
    kr = _sf_rows(k, ue)
    if sfa.dim() != 2 or sfa.shape[0] != kr or sfb.shape != (g, (n + 127) // 128, kr):
        raise ValueError("scale shape mismatch")
    fn = lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0 if ue else lib.dg_m_grouped_fp8_gemm_nt_contiguous
    st = fn(a.data_ptr(), sfa.data_ptr(), _ld(sfa, 0, 4), b.data_ptr(), sfb.data_ptr(), d.data_ptr(), dt,
            m_indices.data_ptr(), m_total, n, k, g, _stream(d))
    _check(st)
    return d


def m_grouped_fp8_gemm_nt_masked(a_pair, b_pair, d: torch.Tensor, masked_m: torch.Tensor,
                                 expected_m: int = 0):
    """Masked-layout M-grouped GEMM; rows at or beyond masked_m[g] are left unwritten."""
    lib = load_library()
    a, sfa = a_pair
    b, sfb = b_pair
    for t, nm in ((a, "a"), (sfa, "sfa"), (b, "b"), (sfb, "sfb"), (d, "d"), (masked_m, "masked_m")):
        _dense_contig(t, nm)
    _fp8(a, "a")
    _fp8(b, "b")
    ue = _sf(sfa, sfb)
    dt = _out(d)
    if masked_m.dtype != torch.int32 or not masked_m.is_cuda:
        raise TypeError("masked_m must be an int32 GPU tensor")
    g, m_max, k = a.shape
    n = b.shape[1]
    if b.shape != (g, n, k) or d.shape != (g, m_max, n) or masked_m.shape != (g,):
        raise ValueError("shape mismatch")
    kr = _sf_rows(k, ue)
    if sfa.dim() != 3 or sfa.shape[:2] != (g, kr) or sfb.shape != (g, (n + 127) // 128, kr):
        raise ValueError("scale shape mismatch")
    fn = lib.dg_m_grouped_fp8_gemm_nt_masked_ue8m0 if ue else lib.dg_m_grouped_fp8_gemm_nt_masked
    # sfa is contiguous [G, rows, L]: the library steps groups by rows * L, so L itself
    # (not a rounded-up stride) is the leading dimension it must validate
    st = fn(a.data_ptr(), sfa.data_ptr(), sfa.shape[2], b.data_ptr(), sfb.data_ptr(), d.data_ptr(), dt,
            masked_m.data_ptr(), g, m_max, n, k, int(expected_m), _stream(d))
    _check(st)
    return d


def _k_grouped_args(a_pair, b_pair, d: torch.Tensor, ks: torch.Tensor):
    a, sfa = a_pair
    b, sfb = b_pair
    for t, nm in ((a, "a"), (b, "b"), (sfb, "sfb"), (d, "d"), (ks, "ks")):
        _dense_contig(t, nm)
    _fp8(a, "a")
    _fp8(b, "b")
    ue = _sf(sfa, sfb)
    if d.dtype != torch.float32 or not d.is_cuda:
        raise TypeError("d must be a float32 GPU tensor")
    if ks.dtype != torch.int32 or not ks.is_cuda:
        raise TypeError("ks must be an int32 GPU tensor")
    m, k = a.shape
    n = b.shape[0]
    g = ks.shape[0]
    if b.shape != (n, k) or d.shape != (g, m, n) or ks.dim() != 1:
        raise ValueError("shape mismatch")
    kr = _sf_rows(k, ue)
    if sfa.dim() != 2 or sfa.shape[0] != kr or sfb.shape != ((n + 127) // 128, kr):
        raise ValueError("scale shape mismatch")
    return a, sfa, b, sfb, g, m, n, k, ue


def k_grouped_fp8_gemm_nt_contiguous(a_pair, b_pair, d: torch.Tensor, ks: torch.Tensor,
                                     c: torch.Tensor | None = None):
    """K-grouped GEMM: D[g] = C[g] + A[:, K_g] @ B[:, K_g].T (FP32), K_g given by ks (int32, device);
    FP32 scales or packed UE8M0 words (int32), by the scale tensors' dtype."""
    lib = load_library()
    a, sfa, b, sfb, g, m, n, k, ue = _k_grouped_args(a_pair, b_pair, d, ks)
    c_ptr = None
    if c is not None:
        if c.dtype != torch.float32 or c.shape != d.shape or not c.is_contiguous() or not c.is_cuda:
            raise ValueError("c must be a contiguous float32 GPU tensor shaped like d")
        c_ptr = c.data_ptr()
    fn = lib.dg_k_grouped_fp8_gemm_nt_contiguous_ue8m0 if ue else lib.dg_k_grouped_fp8_gemm_nt_contiguous
    st = fn(a.data_ptr(), sfa.data_ptr(), _ld(sfa, 0, 4), b.data_ptr(), sfb.data_ptr(), c_ptr, d.data_ptr(),
            ks.data_ptr(), g, m, n, k, _stream(d))
    _check(st)
    return d


def wgrad_fp8_gemm_nt(a_pair, b_pair, d: torch.Tensor, workspace: torch.Tensor | None = None):
    """Dense weight gradient: D += A @ B.T in FP32 (D is read and written).
    ``workspace``: split-K workspace for skinny M (``alloc_workspace``), or None."""
    lib = load_library()
    a, sfa = a_pair
    b, sfb = b_pair
    _fp8(a, "a")
    _fp8(b, "b")
    _f32(sfa, "sfa")
    _f32(sfb, "sfb")
    _dense_contig(sfb, "sfb")
    if d.dtype != torch.float32 or not d.is_cuda or not _unit_last_stride(d):
        raise TypeError("d must be a float32 GPU tensor, contiguous in its last dimension")
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k or d.shape != (m, n):
        raise ValueError("shape mismatch")
    if sfa.dim() != 2 or sfa.shape[0] != k // 128 or sfb.shape != ((n + 127) // 128, k // 128):
        raise ValueError("scale shape mismatch")
    ws, ws_bytes = _workspace(m, n, k, workspace, d)
    st = lib.dg_wgrad_fp8_gemm_nt(a.data_ptr(), _ld(a, 0, 16), sfa.data_ptr(), _ld(sfa, 0, 4), b.data_ptr(),
                                  _ld(b, 0, 16), sfb.data_ptr(), d.data_ptr(), _ld(d, 0, 4), m, n, k, ws, ws_bytes,
                                  _stream(d))
    _check(st)
    return d


def k_grouped_wgrad_fp8_gemm_nt(a_pair, b_pair, d: torch.Tensor, ks: torch.Tensor):
    """K-grouped weight gradient: D[g] += A[:, K_g] @ B[:, K_g].T in FP32."""
    lib = load_library()
    a, sfa, b, sfb, g, m, n, k, ue = _k_grouped_args(a_pair, b_pair, d, ks)
    fn = lib.dg_k_grouped_wgrad_fp8_gemm_nt_ue8m0 if ue else lib.dg_k_grouped_wgrad_fp8_gemm_nt
    st = fn(a.data_ptr(), sfa.data_ptr(), _ld(sfa, 0, 4), b.data_ptr(), sfb.data_ptr(), d.data_ptr(),
            ks.data_ptr(), g, m, n, k, _stream(d))
    _check(st)
    return d


def _cast_args(x: torch.Tensor, q: torch.Tensor, sf: torch.Tensor):
    if x.dtype not in _DTYPES or not x.is_cuda or x.dim() != 2 or not _unit_last_stride(x):
        raise TypeError("x must be a 2-D bfloat16 or float32 GPU tensor, contiguous in its last dimension")
    _fp8(q, "q")
    if q.shape != x.shape:
        raise ValueError("q must have x's shape")
    if sf.dtype not in (torch.float32, torch.int32) or not sf.is_cuda or not _unit_last_stride(sf):
        raise TypeError("sf must be a float32 (FP32 scales) or int32 (packed UE8M0) GPU tensor")
    return _DTYPES[x.dtype], sf.dtype == torch.int32


def per_token_cast_to_fp8(x: torch.Tensor, q: torch.Tensor, sf: torch.Tensor):
    """Per-(row, 128-K) FP8 cast of x [M, K] into q [M, K] and the transposed scales sf:
    FP32 [K/128, ld >= M] or packed UE8M0 int32 [ceil(K/512), ld >= M]."""
    lib = load_library()
    dt, ue = _cast_args(x, q, sf)
    m, k = x.shape
    if sf.dim() != 2 or sf.shape[0] != _sf_rows(k, ue) or sf.shape[1] < m:
        raise ValueError(f"sf shape {tuple(sf.shape)} does not fit x {tuple(x.shape)}")
    st = lib.dg_per_token_cast_to_fp8(x.data_ptr(), _ld(x, 0, 16 // x.element_size()), dt, q.data_ptr(),
                                      _ld(q, 0, 8), sf.data_ptr(), _ld(sf, 0, 4), int(ue), m, k, _stream(x))
    _check(st)
    return q, sf


def per_block_cast_to_fp8(w: torch.Tensor, q: torch.Tensor, sf: torch.Tensor):
    """Per-128x128-block FP8 cast of w [N, K] into q [N, K] and sf: FP32 [ceil(N/128), K/128]
    or packed UE8M0 int32 [ceil(N/128), ceil(K/512)]."""
    lib = load_library()
    dt, ue = _cast_args(w, q, sf)
    n, k = w.shape
    _dense_contig(sf, "sf")
    if sf.shape != ((n + 127) // 128, _sf_rows(k, ue)):
        raise ValueError(f"sf shape {tuple(sf.shape)} does not fit w {tuple(w.shape)}")
    st = lib.dg_per_block_cast_to_fp8(w.data_ptr(), _ld(w, 0, 16 // w.element_size()), dt, q.data_ptr(),
                                      _ld(q, 0, 8), sf.data_ptr(), int(ue), n, k, _stream(w))
    _check(st)
    return q, sf


def fp8_mqa_logits(q: torch.Tensor, kv_pair, weights: torch.Tensor, ks: torch.Tensor, ke: torch.Tensor,
                   clean_logits: bool, out: torch.Tensor):
    """Weighted-ReLU MQA logits: q E4M3 [S, H, D], kv (E4M3 [S_kv, D], FP32 scales [S_kv]),
    weights FP32 [S, H], key ranges ks/ke int32 [S] -> out FP32 [S, S_kv] (caller-allocated)."""
    lib = load_library()
    kv, kv_sf = kv_pair
    for t, nm in ((q, "q"), (kv, "kv"), (kv_sf, "kv_sf"), (weights, "weights"), (ks, "ks"), (ke, "ke")):
        _dense_contig(t, nm)
    _fp8(q, "q")
    _fp8(kv, "kv")
    _f32(kv_sf, "kv_sf")
    _f32(weights, "weights")
    if out.dtype != torch.float32 or not out.is_cuda or not _unit_last_stride(out):
        raise TypeError("out must be a float32 GPU tensor, contiguous in its last dimension")
    for t, nm in ((ks, "ks"), (ke, "ke")):
        if t.dtype != torch.int32 or not t.is_cuda:
            raise TypeError(f"{nm} must be an int32 GPU tensor")
    s, h, d = q.shape
    s_kv = kv.shape[0]
    if kv.shape != (s_kv, d) or kv_sf.shape != (s_kv,) or weights.shape != (s, h) or ks.shape != (s,) \
            or ke.shape != (s,) or out.shape != (s, s_kv):
        raise ValueError("shape mismatch")
    st = lib.dg_fp8_mqa_logits(q.data_ptr(), kv.data_ptr(), kv_sf.data_ptr(), weights.data_ptr(), ks.data_ptr(),
                               ke.data_ptr(), out.data_ptr(), _ld(out, 0, 1), s, s_kv, h, d, int(bool(clean_logits)),
                               _stream(out))
    _check(st)
    return out


def transform_sf_into_required_layout(sf: torch.Tensor, ue8m0: bool = False) -> torch.Tensor:
    """Per-row scales FP32 [mn, kb] (or [G, mn, kb]) -> the GEMM's sfa layout: FP32 [kb, ld]
    (or [G, kb, ld]) transposed with ld = get_sf_aligned_size(mn), or with ``ue8m0`` the packed
    int32 words [ceil(kb/4), ld] holding each scale's exponent byte (powers of two)."""
    lib = load_library()
    if sf.dtype != torch.float32 or not sf.is_cuda or sf.dim() not in (2, 3):
        raise TypeError("sf must be a float32 GPU tensor [mn, kb] or [G, mn, kb]")
    x = sf.contiguous()
    g, mn, kb = (1, *x.shape) if x.dim() == 2 else x.shape
    ld = int(lib.dg_get_sf_aligned_size(mn))
    rows = (kb + 3) // 4 if ue8m0 else kb
    out = torch.empty((g, rows, ld), dtype=torch.int32 if ue8m0 else torch.float32, device=x.device)
    _check(lib.dg_transform_sf_into_required_layout(x.data_ptr(), out.data_ptr(), g, mn, kb, ld,
                                                    1 if ue8m0 else 0, _stream(out)))
    return out[0] if sf.dim() == 2 else out


def get_mn_major_tma_aligned_tensor(sf: torch.Tensor) -> torch.Tensor:
    """Transposed, 16-byte aligned FP32 scales (the README's name for the FP32 form)."""
    return transform_sf_into_required_layout(sf, ue8m0=False)


def get_mn_major_tma_aligned_packed_ue8m0_tensor(sf: torch.Tensor) -> torch.Tensor:
    """Transposed, aligned scales packed into UE8M0 words (scales must be powers of two)."""
    return transform_sf_into_required_layout(sf, ue8m0=True)


def get_mk_alignment_for_contiguous_layout() -> int:
    return load_library().dg_get_mk_alignment_for_contiguous_layout()


def get_sf_aligned_size(mn: int) -> int:
    return load_library().dg_get_sf_aligned_size(mn)


def set_num_cus(n: int):
    _check(load_library().dg_set_num_cus(n))


def get_num_cus() -> int:
    return load_library().dg_get_num_cus()


def _set_tile_n_for_tests(w: int):
    """Force the width of the 256-row tiles (256, 224 or 160; 0 = chosen per call).
    Not part of the API: the tests use it to cover every tile width."""
    _check(load_library().dg_internal_set_tile_n(w))


def _dense_plan_for_tests(m: int, n: int, k: int, cus: int) -> dict:
    """The tile, K split and workspace size a dense call of this shape gets on a
    device with `cus` usable CUs.  Not part of the API: the tests pin the planner."""
    vals = [ctypes.c_int(0) for _ in range(4)]
    ws = ctypes.c_size_t(0)
    _check(load_library().dg_internal_dense_plan(m, n, k, cus, *[ctypes.byref(v) for v in vals], ctypes.byref(ws)))
    bm, bn, splits, sps = (v.value for v in vals)
    return dict(bm=bm, bn=bn, splits=splits, slabs_per_split=sps, ws_bytes=ws.value)


# The README's names for the same utilities ("Utilities": set_num_sms / get_num_sms cap the
# compute units used; get_tma_aligned_size is the aligned leading dimension of the scales).
set_num_sms = set_num_cus
get_num_sms = get_num_cus
get_tma_aligned_size = get_sf_aligned_size
