"""Helpers shared by the GPU tests: upload seeded inputs, call the library
through its binding (which calls the C ABI), read results back.

Sentinels: outputs are pre-filled with a NaN bit pattern so that rows the
library must not write can be checked bit-for-bit afterwards.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import moe_grouped_gemm_tiles_amd as dg

DEV = "cuda:0"
SENT_BF16 = 0x7FBF
SENT_F32 = 0x7FC00123


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def fp8_dev(codes: np.ndarray) -> torch.Tensor:
    return to_dev(codes).view(torch.float8_e4m3fn)


def out_buffer(rows_shape, n: int, dtype: str, ld: int | None = None) -> torch.Tensor:
    """Output pre-filled with the sentinel; optional padded leading dimension."""
    ld = n if ld is None else ld
    shape = tuple(rows_shape) + (ld,)
    if dtype == "bf16":
        t = torch.full(shape, SENT_BF16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    else:
        t = torch.full(shape, SENT_F32, dtype=torch.int32, device=DEV).view(torch.float32)
    return t[..., :n]


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def raw_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy()
    return t.contiguous().view(torch.int32).cpu().numpy()


def sentinel_of(t: torch.Tensor) -> int:
    return np.int16(SENT_BF16) if t.dtype == torch.bfloat16 else np.int32(SENT_F32)


def c_tensor(c: np.ndarray, dtype: str, ld: int | None = None) -> torch.Tensor:
    m, n = c.shape
    t = torch.zeros((m, n if ld is None else ld), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                    device=DEV)
    t[:, :n] = to_dev(c.astype(np.float32)).to(t.dtype)
    return t[:, :n]


def run_dense(x: dict, ld_d: int | None = None, c_in_place: bool = False) -> torch.Tensor:
    a, b = fp8_dev(x["a"]), fp8_dev(x["b"])
    sfa, sfb = to_dev(x["sfa"]), to_dev(x["sfb"])
    if x.get("c") is not None:
        c = c_tensor(x["c"], x["out_dtype"], ld_d)
        if c_in_place:
            d = c
        else:
            d = out_buffer((x["m"],), x["n"], x["out_dtype"], ld_d)
        dg.fp8_gemm_nt((a, sfa), (b, sfb), d, c)
    else:
        d = out_buffer((x["m"],), x["n"], x["out_dtype"], ld_d)
        dg.fp8_gemm_nt((a, sfa), (b, sfb), d)
    torch.cuda.synchronize()
    return d


def run_contiguous(x: dict) -> torch.Tensor:
    d = out_buffer((x["m_total"],), x["n"], x["out_dtype"])
    dg.m_grouped_fp8_gemm_nt_contiguous((fp8_dev(x["a"]), to_dev(x["sfa"])),
                                        (fp8_dev(x["b"]), to_dev(x["sfb"])), d, to_dev(x["m_indices"]))
    torch.cuda.synchronize()
    return d


def run_masked(x: dict, expected_m: int = 0) -> torch.Tensor:
    d = out_buffer((x["num_groups"], x["m_max"]), x["n"], x["out_dtype"])
    dg.m_grouped_fp8_gemm_nt_masked((fp8_dev(x["a"]), to_dev(x["sfa"])),
                                    (fp8_dev(x["b"]), to_dev(x["sfb"])), d, to_dev(x["masked_m"]),
                                    expected_m)
    torch.cuda.synchronize()
    return d


def take(d: torch.Tensor, rows, cols) -> np.ndarray:
    """d[rows][:, cols] as FP64 numpy, gathered on the device."""
    r = torch.as_tensor(np.asarray(rows), device=d.device, dtype=torch.long)
    c = torch.as_tensor(np.asarray(cols), device=d.device, dtype=torch.long)
    return as_f64(d.index_select(0, r).index_select(1, c))


def run_k_grouped(x: dict, with_c: bool = True, in_place: bool = False) -> torch.Tensor:
    """K-grouped GEMM through the binding; D [G, M, N] FP32 pre-filled with the sentinel."""
    a, b = fp8_dev(x["a"]), fp8_dev(x["b"])
    sfa, sfb = to_dev(x["sfa"]), to_dev(x["sfb"])
    ks = to_dev(x["ks"])
    g, m, n = x["num_groups"], x["m"], x["n"]
    if in_place:
        d = to_dev(x["c"].astype(np.float32))
        dg.k_grouped_wgrad_fp8_gemm_nt((a, sfa), (b, sfb), d, ks)
    else:
        d = out_buffer((g, m), n, "fp32")
        c = to_dev(x["c"].astype(np.float32)) if with_c else None
        dg.k_grouped_fp8_gemm_nt_contiguous((a, sfa), (b, sfb), d, ks, c)
    torch.cuda.synchronize()
    return d
