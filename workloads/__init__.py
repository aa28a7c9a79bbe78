"""Seeded synthetic inputs for the fine-grained-scaled FP8 GEMM.

This package produces the bytes and scale factors that both the CPU oracle
(``oracle/``) and the HIP library consume.  It holds no part of the GEMM's
arithmetic: it draws normal FP32 values, quantizes them the way a caller
would before calling the library (an FP8 cast is the caller's job per the
DeepGEMM README, section "Interfaces > Notices", as mirrored on the page
"Weight gradient kernels for dense and MoE models #95"), and lays the
results out in the operand layout the library expects.

Everything here is numpy + torch-CPU; no GPU is touched.
"""

from .gen import (  # noqa: F401
    SF_BLOCK,
    E4M3_MAX,
    quantize_per_row_block,
    quantize_per_block,
    sf_to_mn_major,
    sf_aligned_size,
    pack_ue8m0,
    gen_dense,
    gen_contiguous,
    gen_masked,
    gen_k_grouped,
    gen_quant_input,
    gen_mqa,
    DENSE_SWEEP,
    workload,
    WORKLOAD_NAMES,
)
