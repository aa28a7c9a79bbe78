"""LDS-race check: the debug build of the library (libdg_debug.so, compiled with
a full wait and a workgroup barrier after every phase of LDS traffic) must give
the same bits as the normal library on the tile configurations that stage
operands through LDS: a 256x224 dense GEMM (two 256-row tiles per CU column,
cross-unit prefetch), a split-K skinny GEMM (in-kernel reduction), a 256x256
FP32 GEMM with C and a masked grouped GEMM.  Any difference means the normal
schedule reads a stage before it has landed or overwrites it before every
wave has read it.
"""

import ctypes
import os

import numpy as np
import pytest
import torch

from workloads import gen_dense, gen_masked

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():  # pragma: no cover - GPU only
    import moe_grouped_gemm_tiles_amd as dg
    from tests._gpu_harness import c_tensor, fp8_dev, note, out_buffer, raw_bits, to_dev

DEBUG_LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                         "moe_grouped_gemm_tiles_amd", "libdg_debug.so")


def _libs():
    if not os.path.exists(DEBUG_LIB):
        pytest.fail(f"{DEBUG_LIB} not built (python -m moe_grouped_gemm_tiles_amd.build)")
    debug = ctypes.CDLL(DEBUG_LIB)
    normal = dg.load_library()
    for name in ("dg_fp8_gemm_nt", "dg_m_grouped_fp8_gemm_nt_masked", "dg_get_workspace_size"):
        f, g = getattr(debug, name), getattr(normal, name)
        f.restype, f.argtypes = g.restype, g.argtypes
    return normal, debug


def _dense(lib, x, d, c=None):
    a, sfa, b, sfb = fp8_dev(x["a"]), to_dev(x["sfa"]), fp8_dev(x["b"]), to_dev(x["sfb"])
    m, n, k = x["m"], x["n"], x["k"]
    size = lib.dg_get_workspace_size(m, n, k)
    ws = torch.zeros(max(size, 1) + 256, dtype=torch.uint8, device="cuda:0")
    base = ws.data_ptr() + (-ws.data_ptr()) % 256
    st = lib.dg_fp8_gemm_nt(a.data_ptr(), a.stride(0), sfa.data_ptr(), sfa.stride(0), b.data_ptr(), b.stride(0),
                            sfb.data_ptr(), c.data_ptr() if c is not None else None, c.stride(0) if c is not None else 0,
                            d.data_ptr(), d.stride(0), 0 if d.dtype == torch.bfloat16 else 1, m, n, k,
                            base if size else None, size, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()


@pytest.mark.parametrize("m,n,k,with_c,out", [(4096, 7168, 2048, False, "bf16"),   # 256x224 tiles, 2 rounds
                                              (64, 2112, 7168, False, "bf16"),     # split K, in-kernel reduction
                                              (128, 4096, 7168, True, "fp32"),     # split K with C
                                              (1024, 1024, 4096, True, "fp32")])   # 256x256 with C
def test_dense_debug_build_same_bits(m, n, k, with_c, out):
    normal, debug = _libs()
    x = gen_dense(m, n, k, seed=1600 + m + k, with_c=with_c, out_dtype=out)
    c = c_tensor(x["c"], out) if with_c else None
    d1 = out_buffer((m,), n, out)
    _dense(normal, x, d1, c)
    d2 = out_buffer((m,), n, out)
    _dense(debug, x, d2, c)
    assert np.array_equal(raw_bits(d1), raw_bits(d2)), f"debug build differs: M={m} N={n} K={k}"
    note(f"debug barriers M={m} N={n} K={k} C={with_c}: bit-identical")


def test_masked_debug_build_same_bits():
    normal, debug = _libs()
    x = gen_masked(8, 256, 4096, 2048, seed=1650, masked_m=[256, 0, 17, 200, 129, 64, 255, 1])
    outs = []
    for lib in (normal, debug):
        d = out_buffer((8, 256), 4096, "bf16")
        a, sfa, b, sfb, mm = fp8_dev(x["a"]), to_dev(x["sfa"]), fp8_dev(x["b"]), to_dev(x["sfb"]), to_dev(x["masked_m"])
        st = lib.dg_m_grouped_fp8_gemm_nt_masked(a.data_ptr(), sfa.data_ptr(), sfa.shape[2], b.data_ptr(),
                                                 sfb.data_ptr(), d.data_ptr(), 0, mm.data_ptr(), 8, 256, 4096, 2048,
                                                 128, torch.cuda.current_stream().cuda_stream)
        assert st == 0
        torch.cuda.synchronize()
        outs.append(raw_bits(d))
    assert np.array_equal(outs[0], outs[1])
