"""CPU tests of the dense dispatcher's plan (tile, K split, workspace): host
arithmetic in libdg, reached through its internal test hook."""

import os

import pytest

import moe_grouped_gemm_tiles_amd as dg

CTR_BYTES = 65536
MAX_PARTIALS = 16 << 20


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(dg.library_path()):
        from moe_grouped_gemm_tiles_amd import build
        build.build()
    return dg.load_library()


def cdiv(a, b):
    return -(-a // b)


@pytest.mark.parametrize("m,n,k,want", [
    (128, 7168, 16384, (128, 128, 4, 32)),   # long K: the 128-column tile reads A half as often
    (128, 24576, 1536, (128, 128, 1, 12)),   # enough 128x128 tiles for every CU: no split
    (128, 2112, 7168, (128, 64, 7, 8)),      # few tiles: 64-column tiles, K in 7 splits
    (128, 4096, 7168, (128, 64, 4, 14)),
    (64, 2112, 7168, (64, 128, 8, 7)),
    (1, 7168, 2048, (64, 128, 4, 4)),
    (4096, 7168, 16384, (256, 224, 1, 128)),  # 512 tiles of 256x224 fill two rounds exactly
    (4096, 4096, 7168, (256, 256, 1, 56)),
])
def test_plans_of_the_benchmark_shapes(m, n, k, want):
    p = dg._dense_plan_for_tests(m, n, k, 256)
    assert (p["bm"], p["bn"], p["splits"], p["slabs_per_split"]) == want


@pytest.mark.parametrize("cus", [8, 64, 256])
def test_plan_invariants(cus):
    for m in (1, 33, 64, 65, 100, 128, 129, 4096):
        for n in (13, 300, 1005, 2112, 7168, 24576):
            for k in (128, 512, 1536, 7168, 16384):
                p = dg._dense_plan_for_tests(m, n, k, cus)
                kb = k // 128
                tiles = cdiv(m, p["bm"]) * cdiv(n, p["bn"])
                s, sps = p["splits"], p["slabs_per_split"]
                where = f"M={m} N={n} K={k} cus={cus}: {p}"
                assert (s - 1) * sps < kb <= s * sps, where  # every K block once, no empty split
                if s > 1:
                    assert m <= 128, where  # only skinny GEMMs split K
                    assert tiles * s <= 2 * cus, where
                    assert p["ws_bytes"] == CTR_BYTES + s * tiles * p["bm"] * p["bn"] * 4, where
                    assert p["ws_bytes"] <= CTR_BYTES + MAX_PARTIALS, where
                else:
                    assert p["ws_bytes"] == 0 and sps == kb, where


def test_plan_hook_rejects_bad_sizes(lib):
    import ctypes
    v = [ctypes.c_int(0) for _ in range(4)]
    ws = ctypes.c_size_t(0)
    args = [ctypes.byref(x) for x in v] + [ctypes.byref(ws)]
    for m, n, k, cus in ((0, 256, 512, 256), (64, 0, 512, 256), (64, 256, 500, 256), (64, 256, 512, 0)):
        assert lib.dg_internal_dense_plan(m, n, k, cus, *args) == 1
    assert lib.dg_internal_dense_plan(64, 256, 512, 256, None, None, None, None, None) == 1
