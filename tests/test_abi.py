"""CPU tests of the C ABI: the library loads, exports every symbol the header
declares, and rejects bad arguments synchronously (before touching a GPU)."""

import ctypes
import os
import re

import pytest

import moe_grouped_gemm_tiles_amd as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")

INVALID, UNSUPPORTED = 1, 2


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dg.library_path()):
        from moe_grouped_gemm_tiles_amd import build
        build.build()
    return dg.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_entry_points():
    names = _declared_functions()
    for want in ("dg_fp8_gemm_nt", "dg_m_grouped_fp8_gemm_nt_contiguous", "dg_m_grouped_fp8_gemm_nt_masked",
                 "dg_get_mk_alignment_for_contiguous_layout", "dg_get_sf_aligned_size", "dg_set_num_cus",
                 "dg_get_num_cus", "dg_status_string", "dg_get_workspace_size"):
        assert want in names
    # the configuration surface is the CU cap and DG_PRINT_CONFIGS; tile widths are not part of it
    assert not [n for n in names if "tile_n" in n or "internal" in n]


def test_workspace_size_of_invalid_sizes_is_zero(lib):
    for m, n, k in ((0, 256, 512), (64, 0, 512), (64, 256, 0), (64, 256, 500), (-1, 256, 512)):
        assert lib.dg_get_workspace_size(m, n, k) == 0


def test_library_allocates_nothing():
    """The library source makes no allocation, free or host synchronisation."""
    src = os.path.join(ROOT, "moe_grouped_gemm_tiles_amd", "csrc")
    for f in os.listdir(src):
        text = re.sub(r"//[^\n]*", "", open(os.path.join(src, f)).read())
        for call in ("hipMalloc", "hipFree", "hipStreamSynchronize", "hipDeviceSynchronize", "hipHostMalloc"):
            assert call not in text, (f, call)


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(dg.library_path())
    for name in _declared_functions():
        assert hasattr(raw, name), name


def test_utilities(lib):
    assert lib.dg_get_mk_alignment_for_contiguous_layout() == 128
    assert [lib.dg_get_sf_aligned_size(x) for x in (0, 1, 4, 5, 4096, 33)] == [0, 4, 4, 8, 4096, 36]
    assert lib.dg_get_sf_aligned_size(-1) == -1
    assert lib.dg_set_num_cus(-1) == INVALID
    assert lib.dg_set_num_cus(64) == 0 and lib.dg_get_num_cus() == 64
    assert lib.dg_set_num_cus(0) == 0 and lib.dg_get_num_cus() == 0
    for bad in (-1, 1, 128, 192, 512):
        assert lib.dg_internal_set_tile_n(bad) == INVALID
    for w in (256, 224, 160, 0):
        assert lib.dg_internal_set_tile_n(w) == 0
    for s in range(5):
        assert lib.dg_status_string(s)
    assert lib.dg_status_string(99) == b"DG_UNKNOWN_STATUS"


# Fake, aligned, never-dereferenced addresses: validation fails before any device access.
P = 0x10000


def _dense(lib, **kw):
    args = dict(a=P, lda=512, sfa=P, ld_sfa=128, b=P, ldb=512, sfb=P, c=None, ldc=0, d=P, ldd=256,
                dt=0, m=128, n=256, k=512)
    args.update(kw)
    return lib.dg_fp8_gemm_nt(args["a"], args["lda"], args["sfa"], args["ld_sfa"], args["b"], args["ldb"],
                              args["sfb"], args["c"], args["ldc"], args["d"], args["ldd"], args["dt"],
                              args["m"], args["n"], args["k"], None, 0, None)


def test_dense_validation(lib):
    assert _dense(lib, k=500) == UNSUPPORTED
    assert _dense(lib, m=-1) == INVALID
    assert _dense(lib, dt=7) == INVALID
    assert _dense(lib, a=None) == INVALID
    assert _dense(lib, d=None) == INVALID
    assert _dense(lib, a=P + 8) == INVALID      # 16-byte alignment
    assert _dense(lib, sfa=P + 4) == INVALID
    assert _dense(lib, lda=256) == INVALID      # lda < k
    assert _dense(lib, lda=520) == INVALID      # not a multiple of 16 bytes
    assert _dense(lib, ld_sfa=64) == INVALID    # < M
    assert _dense(lib, ld_sfa=130) == INVALID   # not a multiple of 4
    assert _dense(lib, ldd=100) == INVALID      # < N
    assert _dense(lib, n=250, ldd=250) == INVALID  # BF16 row not 16-byte aligned
    assert _dense(lib, c=P, ldc=100) == INVALID
    assert _dense(lib, c=P + 2, ldc=256) == INVALID
    # empty problems succeed without touching the device
    assert _dense(lib, m=0) == 0
    assert _dense(lib, n=0, ldd=0) == 0


def _contig(lib, **kw):
    args = dict(a=P, sfa=P, ld_sfa=256, b=P, sfb=P, d=P, dt=0, mi=P, m=256, n=256, k=512, g=4)
    args.update(kw)
    return lib.dg_m_grouped_fp8_gemm_nt_contiguous(args["a"], args["sfa"], args["ld_sfa"], args["b"], args["sfb"],
                                                   args["d"], args["dt"], args["mi"], args["m"], args["n"],
                                                   args["k"], args["g"], None)


def test_contiguous_validation(lib):
    assert _contig(lib, m=200, ld_sfa=200) == UNSUPPORTED  # M_total % 128
    assert _contig(lib, k=100) == UNSUPPORTED
    assert _contig(lib, g=-1) == INVALID
    assert _contig(lib, mi=None) == INVALID
    assert _contig(lib, mi=P + 2) == INVALID
    assert _contig(lib, ld_sfa=128) == INVALID
    assert _contig(lib, n=100) == INVALID  # BF16 rows must stay 16-byte aligned
    assert _contig(lib, m=0, ld_sfa=0) == 0
    assert _contig(lib, g=0) == 0


def _masked(lib, **kw):
    args = dict(a=P, sfa=P, ld_sfa=256, b=P, sfb=P, d=P, dt=1, mm=P, g=4, mmax=256, n=256, k=512, em=0)
    args.update(kw)
    return lib.dg_m_grouped_fp8_gemm_nt_masked(args["a"], args["sfa"], args["ld_sfa"], args["b"], args["sfb"],
                                               args["d"], args["dt"], args["mm"], args["g"], args["mmax"],
                                               args["n"], args["k"], args["em"], None)


def test_masked_validation(lib):
    assert _masked(lib, k=130) == UNSUPPORTED
    assert _masked(lib, g=-2) == INVALID
    assert _masked(lib, mm=None) == INVALID
    assert _masked(lib, ld_sfa=100) == INVALID
    assert _masked(lib, b=P + 1) == INVALID
    assert _masked(lib, n=2, dt=1) == INVALID  # FP32 rows of 8 bytes
    assert _masked(lib, mmax=0) == 0
    assert _masked(lib, g=0) == 0


def test_binding_refuses_cpu_tensors(lib):
    import torch
    a = torch.zeros(128, 128, dtype=torch.uint8)
    s = torch.ones(1, 128)
    d = torch.zeros(128, 128, dtype=torch.bfloat16)
    with pytest.raises((TypeError, ValueError)):
        dg.fp8_gemm_nt((a, s), (a, s), d)


def test_header_declares_next_entry_points():
    names = _declared_functions()
    for want in ("dg_fp8_gemm_nt_ue8m0", "dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0",
                 "dg_m_grouped_fp8_gemm_nt_masked_ue8m0", "dg_k_grouped_fp8_gemm_nt_contiguous",
                 "dg_wgrad_fp8_gemm_nt", "dg_k_grouped_wgrad_fp8_gemm_nt"):
        assert want in names


def test_ue8m0_validation(lib):
    f = lib.dg_fp8_gemm_nt_ue8m0
    ok = (P, 512, P, 128, P, 512, P, None, 0, P, 256, 0, 128, 256, 512, None, 0, None)
    bad_ld = list(ok)
    bad_ld[3] = 130  # ld_sfa not a multiple of 4 words
    assert f(*bad_ld) == INVALID
    bad_k = list(ok)
    bad_k[14] = 500
    assert f(*bad_k) == UNSUPPORTED
    empty = list(ok)
    empty[12] = 0
    assert f(*empty) == 0
    g = lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0
    assert g(P, P, 256, P, P, P, 0, None, 256, 256, 512, 4, None) == INVALID  # no m_indices
    h = lib.dg_m_grouped_fp8_gemm_nt_masked_ue8m0
    assert h(P, P, 100, P, P, P, 0, P, 4, 256, 256, 512, 0, None) == INVALID  # ld_sfa < m_max


def _kg(lib, **kw):
    args = dict(a=P, sfa=P, ld_sfa=256, b=P, sfb=P, c=None, d=P, ks=P, g=4, m=256, n=256, k=1024)
    args.update(kw)
    return lib.dg_k_grouped_fp8_gemm_nt_contiguous(args["a"], args["sfa"], args["ld_sfa"], args["b"], args["sfb"],
                                                   args["c"], args["d"], args["ks"], args["g"], args["m"],
                                                   args["n"], args["k"], None)


def test_k_grouped_and_wgrad_validation(lib):
    assert _kg(lib, k=1000) == UNSUPPORTED
    assert _kg(lib, g=-1) == INVALID
    assert _kg(lib, ks=None) == INVALID
    assert _kg(lib, ks=P + 2) == INVALID
    assert _kg(lib, c=P + 4) == INVALID
    assert _kg(lib, n=3) == INVALID    # FP32 rows of 12 bytes
    assert _kg(lib, ld_sfa=100) == INVALID
    assert _kg(lib, m=0) == 0 and _kg(lib, g=0) == 0
    w = lib.dg_wgrad_fp8_gemm_nt
    assert w(P, 512, P, 128, P, 512, P, P, 100, 128, 256, 512, None, 0, None) == INVALID  # ldd < n
    assert w(P, 512, P, 128, P, 512, P, P, 256, 0, 256, 512, None, 0, None) == 0
    kw = lib.dg_k_grouped_wgrad_fp8_gemm_nt
    assert kw(P, P, 256, P, P, P, None, 4, 256, 256, 1024, None) == INVALID  # no ks
    ku = lib.dg_k_grouped_fp8_gemm_nt_contiguous_ue8m0
    assert ku(P, P, 256, P, P, None, P, P, 4, 256, 256, 1000, None) == UNSUPPORTED  # k % 128
    assert ku(P, P, 100, P, P, None, P, P, 4, 256, 256, 1024, None) == INVALID      # ld_sfa < m
    assert ku(P, P, 256, P, P, None, P, P, 0, 256, 256, 1024, None) == 0
    kwu = lib.dg_k_grouped_wgrad_fp8_gemm_nt_ue8m0
    assert kwu(P, P, 256, P, P, P, None, 4, 256, 256, 1024, None) == INVALID  # no ks


def test_binding_leading_dimension_of_size_one_dims():
    import torch
    from moe_grouped_gemm_tiles_amd import _ld
    t = torch.zeros(1, 4, dtype=torch.int32).as_strided((1, 4), (1, 1))  # any stride is legal for a size-1 dim
    assert _ld(t, 0, 4) == 4
    assert _ld(torch.zeros(1, 6), 0, 4) == 8
    assert _ld(torch.zeros(3, 1, 5), 1, 4) == 8
    assert _ld(torch.zeros(5, 7)[:, :3], 0, 4) == 7
