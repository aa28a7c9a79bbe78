"""CPU oracle for the fine-grained-scaled FP8 GEMM.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding)
never imports, links or calls it, and shares no code with it: no kernels,
tables, helpers or constants.  Inputs reach both sides from ``workloads/``.

What it computes, written out plainly in FP64 with numpy:

* an E4M3 decode table built from the format's closed form (``e4m3.py``);
* dense ``D = C + A @ B.T`` in NT layout with per-(row, 128-K) FP32 scales on
  A and per-128x128-block FP32 scales on B (``gemm.py``);
* the M-grouped contiguous and masked variants as per-group dense GEMMs,
  reporting which rows the library must leave unwritten (``gemm.py``);
* UE8M0 (power-of-two, packed four per word) scale factors and the three
  GEMM variants with them (``ue8m0.py``);
* the K-grouped GEMM of the MoE weight gradient (``kgrouped.py``);
* the FP8 quantization a caller performs before the GEMM, per-token 1x128
  and per-block 128x128, FP32 or UE8M0 scales (``quant.py``);
* the weighted-ReLU MQA logits of the indexer (``mqa.py``);
* the scale-factor layout transform: per-row scales to the transposed,
  aligned FP32 form or the packed UE8M0 form (``layout.py``);
* the acceptance check (``check.py``).

Sources, by page title and section:

* DeepGEMM README as mirrored on the page "Weight gradient kernels for dense
  and MoE models #95": "Interfaces > Notices" (D = C + A @ B.T, NT layout,
  FP32 scale factors on SM90, transposed LHS scale layout), "Grouped GEMMs
  (contiguous layout)" (M-only grouping, segments aligned to the M block),
  "Grouped GEMMs (masked layout)" (a mask tensor; only valid parts computed).
* GeekNews digest "DeepGEMM: बारीक scaling के जरिए साफ़ और efficient FP8 GEMM
  kernel": section "GEMM interface और layout constraints" (same interface
  facts) and the Hacker News comments on promotion of MMA partial sums into
  FP32 accumulators.
* Same README, sections "Grouped GEMMs (contiguous layout)" (the K-axis
  grouped API for the MoE weight backward), "V3.2 MQA kernels for the
  indexer" (the logits formula), "Utilities" (scale-factor layout helpers,
  packed UE8M0); the pull-request text on that page (FP8 x FP8 -> FP32
  weight-gradient GEMMs).

Every function is pinned by tests under ``tests/`` marked ``not gpu``
(closed forms, brute force in exact rationals, one-hot products, scale
linearity, grouped-equals-dense, K groups summing to the dense product,
torch's independent E4M3 / E8M0 decoders and E4M3 cast, ReLU and weight
properties of the MQA logits).  No function here is "parity unpinned".
"""

from .e4m3 import E4M3_TABLE, e4m3_closed_form, decode_e4m3  # noqa: F401
from .gemm import (  # noqa: F401
    dequant_a,
    dequant_b,
    ref_dense,
    ref_contiguous,
    ref_masked,
)
from .ue8m0 import (  # noqa: F401
    UE8M0_TABLE,
    unpack_ue8m0,
    decode_ue8m0_sf,
    ref_dense_ue8m0,
    ref_contiguous_ue8m0,
    ref_k_grouped_ue8m0,
    ref_masked_ue8m0,
)
from .kgrouped import k_offsets, ref_k_grouped  # noqa: F401
from .quant import e4m3_encode_rne, quant_per_token, quant_per_block  # noqa: F401
from .mqa import ref_mqa_logits  # noqa: F401
from .layout import transform_sf  # noqa: F401
from .check import tolerance_report, assert_close, TOL_REL, TOL_RMS, TOL_COS  # noqa: F401
