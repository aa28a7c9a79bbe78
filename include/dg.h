/*
 * dg.h -- C ABI of libdg: fine-grained-scaled FP8 GEMM for AMD Instinct
 * MI355X (gfx950, CDNA4).
 *
 * Computes D = C + A @ B.T in NT layout (A row-major [M,K], B row-major
 * [N,K], i.e. both K-contiguous) where A and B hold OCP E4M3 (E4M3FN) byte
 * codes, A carries one FP32 (or UE8M0) scale per (row, 128-wide K block) and
 * B one per 128x128 block; plus the K-grouped / weight-gradient GEMMs, the FP8
 * cast that produces the operands, and the MQA logits of the indexer.
 * Sources, by page title and section:
 *
 *   [README]  DeepGEMM README as mirrored on the page "Weight gradient
 *             kernels for dense and MoE models #95" (English); the same text
 *             is summarised on the GeekNews page "DeepGEMM: बारीक scaling के
 *             जरिए साफ़ और efficient FP8 GEMM kernel".
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library keeps no pointer after the call returns.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream).
 *     Nothing synchronises with the host and the library allocates no
 *     memory, so every entry point may be captured into a HIP graph.
 *   - Scale layouts:
 *       sfa: FP32 [K/128][ld_sfa], transposed ("MN-major"): sfa[kb*ld_sfa + m]
 *            scales A[m, kb*128 .. kb*128+127].  ld_sfa >= rows of A and
 *            ld_sfa % 4 == 0 (16-byte rows), see dg_get_sf_aligned_size.
 *            ([README] "Interfaces > Notices": the LHS scale factor is FP32
 *            on SM90-class parts and must be in a transposed, aligned layout.)
 *       sfb: FP32 [ceil(N/128)][K/128] row-major: sfb[nb*(K/128) + kb] scales
 *            B[nb*128 .. nb*128+127, kb*128 .. kb*128+127] (the last row
 *            block may be partial when N % 128 != 0).
 *   - Accumulation: each 128-K slab's FP8 product is computed on the matrix
 *     cores, scaled by sfa*sfb and added into FP32 accumulators; C (if any)
 *     is added in FP32 and D is rounded once (BF16: round to nearest even).
 *   - Determinism: for a fixed shape and device CU count, repeated calls
 *     give bit-identical D (no floating-point atomics; fixed reduction order).
 *   - Errors: argument problems are reported synchronously before anything
 *     is enqueued.  Data that lives on the device (group indices, masks) is
 *     never an error: out-of-range values are clamped or skipped so that all
 *     memory accesses stay in bounds.
 *
 * Workspace: skinny dense GEMMs (M <= 128) may split K across workgroups (the
 * library decides per shape and CU count; a call splits exactly when
 * dg_get_workspace_size is not 0).  Each workgroup writes the FP32 partial sum of its K range to a
 * caller-owned workspace and counts itself in a per-tile counter there; the
 * workgroup that completes a tile adds the partials in K-range order (so the
 * result is deterministic), writes D and resets the counter.  One launch per
 * call.  The workspace:
 *   - size: dg_get_workspace_size(m, n, k) bytes (0 = the call needs none and
 *     may pass NULL); the size depends on the shape and on the CU count in use
 *     (dg_set_num_cus), so query it with the same settings as the call;
 *   - device memory, 256-byte aligned, ZERO-FILLED before its first use; every
 *     call leaves it ready for the next one (its counters back at zero), so it
 *     is cleared once, not per call;
 *   - owned by the caller: the library keeps no pointer to it.  Calls that
 *     share one workspace must not overlap (order them on one stream); calls
 *     on concurrent streams need workspaces of their own.
 * A missing, misaligned or too small workspace -> DG_ERROR_WORKSPACE.
 */
#ifndef DG_H
#define DG_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DG_SUCCESS = 0,
  DG_ERROR_INVALID_VALUE = 1,  /* null/misaligned pointer, bad stride, negative size, bad enum */
  DG_ERROR_NOT_SUPPORTED = 2,  /* valid but unsupported: K % 128 != 0, contiguous M % 128 != 0 */
  DG_ERROR_LAUNCH_FAILED = 3,  /* a HIP call failed; hipGetLastError() text via dg_last_hip_error */
  DG_ERROR_WORKSPACE = 4,      /* split-K workspace NULL, misaligned or smaller than dg_get_workspace_size */
  DG_ERROR_SCRATCH_LIMIT = 5   /* dg_fp8_gemm_nt_noalloc: the call needs more than the library's fixed scratch */
} dg_status;

typedef enum { DG_DTYPE_BF16 = 0, DG_DTYPE_FP32 = 1 } dg_dtype;

/*
 * Dense GEMM: D[M,N] = C[M,N] + A[M,K] @ B[N,K]^T.
 *   [README] "Interfaces > Notices" (fp8_gemm_nt computes D = C + A @ B.T) and
 *   "Normal dense GEMMs (non-grouped)".
 *
 * a      E4M3 bytes, row m at a + m*lda; lda >= k, lda % 16 == 0, a 16-B aligned.
 * sfa    FP32 [k/128][ld_sfa] as above; ld_sfa >= m, ld_sfa % 4 == 0, 16-B aligned.
 * b      E4M3 bytes, row n at b + n*ldb; ldb >= k, ldb % 16 == 0, 16-B aligned.
 * sfb    FP32 [ceil(n/128)][k/128], 4-B aligned.
 * c      optional (NULL = no C); same dtype as d; row stride ldc elements,
 *        ldc >= n, rows 16-B aligned.  c may equal d (in-place accumulate);
 *        any other overlap of c and d is undefined.
 * d      output, dtype d_dtype, row stride ldd elements, ldd >= n, rows 16-B aligned.
 * m,n,k  sizes; m == 0 or n == 0 -> DG_SUCCESS with nothing enqueued;
 *        k == 0 -> D = C (or 0); k % 128 != 0 -> DG_ERROR_NOT_SUPPORTED.
 * workspace, workspace_bytes
 *        split-K workspace (see "Workspace" above); NULL and 0 when
 *        dg_get_workspace_size(m, n, k) is 0.
 */
dg_status dg_fp8_gemm_nt(const void* a, int64_t lda, const float* sfa, int64_t ld_sfa,
                         const void* b, int64_t ldb, const float* sfb,
                         const void* c, int64_t ldc, void* d, int64_t ldd, dg_dtype d_dtype,
                         int m, int n, int k, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * Allocation-free form of dg_fp8_gemm_nt, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same computation, kernels and bits as
 * dg_fp8_gemm_nt with a workspace, but the split-K scratch is a fixed array
 * inside the library (64 KiB of counters + 16 MiB of partial tiles on each
 * device, held from the library's first use on that device until the process
 * ends).  No memory is allocated or freed by the call.
 *   - Every call on a device shares that device's scratch: calls that overlap
 *     on one device (other streams, other host threads) RACE and may return
 *     wrong results; order them (one stream).
 *   - Each split call first clears the counters it uses (one small kernel on
 *     `stream`), so a call does not depend on what the previous one left.
 *   - A call that needs more scratch than the fixed size ->
 *     DG_ERROR_SCRATCH_LIMIT, nothing enqueued.  Every dense plan keeps its
 *     partials within 16 MiB, so with these kernels this does not happen.
 * Arguments, layouts and other errors as for dg_fp8_gemm_nt.
 */
dg_status dg_fp8_gemm_nt_noalloc(const void* a, int64_t lda, const float* sfa, int64_t ld_sfa,
                                 const void* b, int64_t ldb, const float* sfb,
                                 const void* c, int64_t ldc, void* d, int64_t ldd, dg_dtype d_dtype,
                                 int m, int n, int k, hipStream_t stream);

/*
 * Bytes of split-K workspace the dense GEMMs (dg_fp8_gemm_nt, its UE8M0 form
 * and dg_wgrad_fp8_gemm_nt) need for an M x N x K call on the current device
 * with the current CU cap (at most 64 KiB + 16 MiB); 0 when the call does not
 * split K (always for M > 128) or the sizes are invalid.  One workspace serves calls of several shapes
 * if it is at least as large as each call's size.  Host-only, enqueues nothing.
 *   (The pages leave the workspace of split reductions unspecified; the
 *   README's calls take caller-allocated outputs, "Mega MoE" usage.)
 */
size_t dg_get_workspace_size(int m, int n, int k);

/*
 * M-grouped GEMM, contiguous layout (MoE prefill / training forward):
 *   [README] "Grouped GEMMs (contiguous layout)": only M is grouped, N and K
 *   are shared by all groups; tokens of all experts are concatenated and each
 *   expert segment is aligned to the M block (dg_get_mk_alignment_for_contiguous_layout).
 *
 * a          E4M3 [m_total, k] contiguous (row stride k).
 * sfa        FP32 [k/128][ld_sfa], ld_sfa >= m_total, ld_sfa % 4 == 0.
 * b          E4M3 [num_groups, n, k] contiguous.
 * sfb        FP32 [num_groups][ceil(n/128)][k/128] contiguous.
 * d          [m_total, n] contiguous, dtype d_dtype.
 * m_indices  DEVICE int32 [m_total]: group of each row, -1 on padding rows.
 *            Row r is computed with group m_indices[r]'s B.  Rows whose index
 *            is outside [0, num_groups) are NOT written.  The group of a
 *            128-row block is read from its first row; a block that mixes
 *            groups breaks the layout contract (rows of other groups are
 *            left unwritten, never out of bounds).
 * m_total % 128 != 0 -> DG_ERROR_NOT_SUPPORTED.
 * The call enqueues one kernel, or two on the same stream when the last round
 * of 256-row tiles would keep at most half the CUs busy (its rows then go to
 * 128x128 tiles; same bits).
 */
dg_status dg_m_grouped_fp8_gemm_nt_contiguous(const void* a, const float* sfa, int64_t ld_sfa,
                                              const void* b, const float* sfb,
                                              void* d, dg_dtype d_dtype,
                                              const int32_t* m_indices,
                                              int m_total, int n, int k, int num_groups,
                                              hipStream_t stream);

/*
 * M-grouped GEMM, masked layout (MoE decode under graph capture):
 *   [README] "Grouped GEMMs (masked layout)": the host does not know each
 *   expert's token count; a mask tensor tells the kernel which parts are
 *   valid and only those are computed.
 *
 * a          E4M3 [num_groups, m_max, k] contiguous.
 * sfa        FP32 [num_groups][k/128][ld_sfa], ld_sfa >= m_max, ld_sfa % 4 == 0.
 * b          E4M3 [num_groups, n, k] contiguous.
 * sfb        FP32 [num_groups][ceil(n/128)][k/128] contiguous.
 * d          [num_groups, m_max, n] contiguous, dtype d_dtype.
 * masked_m   DEVICE int32 [num_groups]: valid rows of each group, clamped to
 *            [0, m_max].  Rows at or beyond it are NOT written.
 * expected_m host hint of the typical masked_m (<= 0: unknown); used only to
 *            choose tile sizes, never as data.
 */
dg_status dg_m_grouped_fp8_gemm_nt_masked(const void* a, const float* sfa, int64_t ld_sfa,
                                          const void* b, const float* sfb,
                                          void* d, dg_dtype d_dtype,
                                          const int32_t* masked_m,
                                          int num_groups, int m_max, int n, int k,
                                          int expected_m, hipStream_t stream);

/*
 * UE8M0 variants of the three GEMMs above.  [README] "Interfaces > Notices":
 * the newer architecture takes UE8M0 scale factors, four packed into one
 * 32-bit integer, instead of FP32.  Same granularity as the FP32 form (A per
 * (row, 128-K block), B per 128x128 block); each byte e means 2^(e-127), 255
 * is NaN.  Packing runs along K: byte j (least significant first) of word q
 * holds the scale of K block 4q + j; bytes past the last K block are ignored.
 * On gfx950 the scales feed the MFMA's block-scale operands, so the K loop
 * accumulates in the matrix core without FP32 promotion.
 *
 * sfa   int32 words [ceil(k/512)][ld_sfa] (masked: [num_groups][ceil(k/512)][ld_sfa]),
 *       ld_sfa >= rows of A, ld_sfa % 4 == 0, 16-B aligned.
 * sfb   int32 words [ceil(n/128)][ceil(k/512)] (grouped: [num_groups][...]), 4-B aligned.
 * All other arguments, layouts and errors as in the FP32-scale entry points.
 */
dg_status dg_fp8_gemm_nt_ue8m0(const void* a, int64_t lda, const int32_t* sfa, int64_t ld_sfa,
                               const void* b, int64_t ldb, const int32_t* sfb,
                               const void* c, int64_t ldc, void* d, int64_t ldd, dg_dtype d_dtype,
                               int m, int n, int k, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);
dg_status dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(const void* a, const int32_t* sfa, int64_t ld_sfa,
                                                    const void* b, const int32_t* sfb,
                                                    void* d, dg_dtype d_dtype,
                                                    const int32_t* m_indices,
                                                    int m_total, int n, int k, int num_groups,
                                                    hipStream_t stream);
dg_status dg_m_grouped_fp8_gemm_nt_masked_ue8m0(const void* a, const int32_t* sfa, int64_t ld_sfa,
                                                const void* b, const int32_t* sfb,
                                                void* d, dg_dtype d_dtype,
                                                const int32_t* masked_m,
                                                int num_groups, int m_max, int n, int k,
                                                int expected_m, hipStream_t stream);

/*
 * K-grouped GEMM (MoE weight gradient):
 *   [README] "Grouped GEMMs (contiguous layout)": a K-axis-grouped API for the
 *   MoE weight backward, with M and N fixed; the pull-request text on the
 *   same page: FP8 x FP8 -> FP32 weight-gradient GEMMs for dense and MoE models.
 *
 * Group g owns K range [k_off[g], k_off[g] + ks[g]) where k_off is the
 * exclusive prefix sum of ks, and D[g] = C[g] + A[:, range] @ B[:, range]^T.
 *
 * a        E4M3 [m, k_total] contiguous (row stride k_total): K-contiguous ("NT");
 *          token-major tensors are transposed by the caller.
 * sfa      FP32 [k_total/128][ld_sfa], ld_sfa >= m, ld_sfa % 4 == 0 (scales by
 *          global K block).
 * b        E4M3 [n, k_total] contiguous.
 * sfb      FP32 [ceil(n/128)][k_total/128].
 * c        optional FP32 [num_groups, m, n] contiguous (NULL = zero); may equal d.
 * d        FP32 [num_groups, m, n] contiguous.  Every group's D is written, also
 *          for ks[g] == 0 (then D[g] = C[g] or 0).
 * ks       DEVICE int32 [num_groups]: K size of each group, a multiple of 128
 *          (dg_get_mk_alignment_for_contiguous_layout).  Device data is clamped,
 *          never an error: negative sizes count as 0, sizes round down to a
 *          multiple of 128, and ranges past k_total are cut at k_total.
 * k_total  sum of ks; k_total % 128 != 0 -> DG_ERROR_NOT_SUPPORTED.
 */
dg_status dg_k_grouped_fp8_gemm_nt_contiguous(const void* a, const float* sfa, int64_t ld_sfa,
                                              const void* b, const float* sfb,
                                              const float* c, float* d, const int32_t* ks,
                                              int num_groups, int m, int n, int k_total,
                                              hipStream_t stream);

/*
 * Weight-gradient GEMMs with FP32 accumulation in place (the pull request on
 * the page "Weight gradient kernels for dense and MoE models #95"):
 *   dg_wgrad_fp8_gemm_nt            D[m,n] += A[m,k] @ B[n,k]^T           (dense)
 *   dg_k_grouped_wgrad_fp8_gemm_nt  D[g]   += A[:, K_g] @ B[:, K_g]^T      (K-grouped)
 * They are dg_fp8_gemm_nt with c = d (FP32) and dg_k_grouped_fp8_gemm_nt_contiguous
 * with c = d; arguments as there (the dense one takes the split-K workspace).
 */
dg_status dg_wgrad_fp8_gemm_nt(const void* a, int64_t lda, const float* sfa, int64_t ld_sfa,
                               const void* b, int64_t ldb, const float* sfb,
                               float* d, int64_t ldd, int m, int n, int k,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);
dg_status dg_k_grouped_wgrad_fp8_gemm_nt(const void* a, const float* sfa, int64_t ld_sfa,
                                         const void* b, const float* sfb, float* d, const int32_t* ks,
                                         int num_groups, int m, int n, int k_total, hipStream_t stream);

/*
 * The two K-grouped GEMMs above with packed UE8M0 scale factors.
 *   [README] "Utilities": a K-grouped GEMM packing kernel for MN-major
 *   UE8M0 scales; "Interfaces > Notices": UE8M0 scales packed four per int.
 * sfa  int32 words [ceil(k_total/512)][ld_sfa]: byte j (least significant
 *      first) of word q scales A's global K block 4q + j (2^(byte-127)).
 * sfb  int32 words [ceil(n/128)][ceil(k_total/512)], same packing along K.
 * Words are packed along the global K blocks, so a word may hold blocks of
 * two adjacent groups (group ranges are multiples of 128, not of 512).
 * Everything else as for the FP32-scale forms.
 */
dg_status dg_k_grouped_fp8_gemm_nt_contiguous_ue8m0(const void* a, const int32_t* sfa, int64_t ld_sfa,
                                                    const void* b, const int32_t* sfb, const float* c, float* d,
                                                    const int32_t* ks, int num_groups, int m, int n, int k_total,
                                                    hipStream_t stream);
dg_status dg_k_grouped_wgrad_fp8_gemm_nt_ue8m0(const void* a, const int32_t* sfa, int64_t ld_sfa, const void* b,
                                               const int32_t* sfb, float* d, const int32_t* ks, int num_groups,
                                               int m, int n, int k_total, hipStream_t stream);

/*
 * FP8 quantization of GEMM operands (the cast the GEMM's caller performs,
 * [README] "Interfaces > Notices": FP8 casting and transposition are the
 * caller's job, and the LHS scale factors must be transposed and aligned;
 * "Utilities": helpers producing those scale layouts, FP32 or packed UE8M0).
 *
 * Scale rule: FP32 s = amax / 448 (computed in FP32; 1 for an all-zero
 * block); UE8M0 s = the smallest power of two >= fp32(amax / 448) (1 for an
 * all-zero block), stored as the byte log2(s) + 127.  Codes are
 * E4M3(clamp(x / s, -448, 448)): the quotient correctly rounded to FP32, then
 * rounded to E4M3 with ties to even.  Inputs must be finite (codes of NaN or
 * Inf inputs are unspecified).
 *
 * dg_per_token_cast_to_fp8: x [m, k] (BF16 or FP32, row stride ldx elements,
 *   16-B aligned rows) -> q E4M3 [m, k] (row stride ldq bytes, ldq % 8 == 0)
 *   and sf, one scale per (row, 128-K block), stored transposed: FP32
 *   [k/128][ld_sf] or (ue8m0 != 0) int32 words [ceil(k/512)][ld_sf], four
 *   bytes per word along K (padding bytes 127); ld_sf >= m, ld_sf % 4 == 0,
 *   sf 16-B aligned.  Columns m..ld_sf-1 of sf are not written.  This is the
 *   sfa operand of the GEMM entry points.
 * dg_per_block_cast_to_fp8: w [n, k] -> q [n, k] and sf, one scale per
 *   128 x 128 block: FP32 [ceil(n/128)][k/128] or int32 words
 *   [ceil(n/128)][ceil(k/512)] (padding bytes 127).  This is the sfb operand.
 * k % 128 != 0 -> DG_ERROR_NOT_SUPPORTED; m (n) == 0 or k == 0 -> DG_SUCCESS.
 */
dg_status dg_per_token_cast_to_fp8(const void* x, int64_t ldx, dg_dtype x_dtype, void* q, int64_t ldq,
                                   void* sf, int64_t ld_sf, int ue8m0, int m, int k, hipStream_t stream);
dg_status dg_per_block_cast_to_fp8(const void* w, int64_t ldw, dg_dtype w_dtype, void* q, int64_t ldq,
                                   void* sf, int ue8m0, int n, int k, hipStream_t stream);

/*
 * Weighted-ReLU MQA logits (the lightning-indexer scoring kernel, non-paged).
 *   [README] "V3.2 MQA kernels for the indexer": for query i and each key j
 *   in [ks[i], ke[i]),
 *     out[i, j] = sum_h weights[i, h] * relu( q[i, h, :] . kv[j, :] * kv_sf[j] ),
 *   positions outside the range are set to -inf when clean_logits != 0.
 *
 * q        E4M3 [s, num_heads, head_dim] contiguous, 16-B aligned (no scale).
 * kv       E4M3 [s_kv, head_dim] contiguous, 16-B aligned.
 * kv_sf    FP32 [s_kv], one scale per kv row; must be >= 0 (a quantization
 *          scale; the kernel applies it after the ReLU).
 * weights  FP32 [s, num_heads] contiguous, 16-B aligned.
 * ks, ke   DEVICE int32 [s]: key range of each query, clamped to [0, s_kv];
 *          an empty range writes no logit.
 * out      FP32 [s, ld_out], ld_out >= s_kv.  Without clean_logits the
 *          positions outside each range are left untouched.
 * head_dim must be 128 and num_heads a multiple of 16 up to 64
 * (else DG_ERROR_NOT_SUPPORTED); s == 0 or s_kv == 0 -> DG_SUCCESS.
 */
dg_status dg_fp8_mqa_logits(const void* q, const void* kv, const float* kv_sf, const float* weights,
                            const int32_t* ks, const int32_t* ke, float* out, int64_t ld_out,
                            int s, int s_kv, int num_heads, int head_dim, int clean_logits,
                            hipStream_t stream);

/*
 * Scale-factor layout transform.
 *   [README] "Utilities": transform_sf_into_required_layout,
 *   get_mn_major_tma_aligned_tensor and
 *   get_mn_major_tma_aligned_packed_ue8m0_tensor; "Interfaces > Notices": the
 *   LHS scale factor is transposed and aligned, and the UE8M0 form packs four
 *   scale bytes into one int.
 *
 * sf      DEVICE FP32 [num_groups][mn][kb] row-major per-row scales (one per
 *         row and 128-wide K block), 4-B aligned.
 * out     DEVICE, 16-B aligned, caller-allocated:
 *           ue8m0 == 0: FP32 [num_groups][kb][ld_out], out[g][k][r] = sf[g][r][k];
 *           ue8m0 != 0: int32 [num_groups][ceil(kb/4)][ld_out]; byte j (least
 *             significant first) of out[g][q][r] is the biased exponent field
 *             (bits 30..23) of sf[g][r][4q+j] -- exactly the UE8M0 code when
 *             the scale is a power of two -- and 127 where 4q+j >= kb.
 *         Columns mn..ld_out-1 are not written.
 * ld_out  >= mn and a multiple of 4 (dg_get_sf_aligned_size(mn)), else
 *         DG_ERROR_INVALID_VALUE.  The result is the sfa operand of the GEMM
 *         entry points (masked: one group per expert).
 * num_groups, mn or kb == 0 -> DG_SUCCESS with nothing enqueued; more than
 * 65535 groups -> DG_ERROR_NOT_SUPPORTED.
 */
dg_status dg_transform_sf_into_required_layout(const float* sf, void* out, int num_groups, int mn, int kb,
                                               int64_t ld_out, int ue8m0, hipStream_t stream);

/* Row (M-grouped) and K (K-grouped) alignment of group segments in the
 * contiguous layouts (128).
 * [README] "Utilities": get_mk_alignment_for_contiguous_layout. */
int dg_get_mk_alignment_for_contiguous_layout(void);

/* Leading dimension (in floats) for a transposed FP32 scale tensor with mn
 * rows: mn rounded up to 4 (16 bytes).  Returns -1 for mn < 0.
 * [README] "Utilities": get_tma_aligned_size. */
int64_t dg_get_sf_aligned_size(int64_t mn);

/* Cap on compute units the kernels spread over (0 = all CUs of the current
 * device, the default; DG_NUM_CUS in the environment sets the initial value).
 * Negative -> DG_ERROR_INVALID_VALUE.  Process-wide.  dg_get_num_cus returns
 * the CUs the kernels use on the current device (the cap, or all CUs when
 * uncapped); without a usable device it returns the cap (0 = uncapped).
 * [README] "Utilities": set_num_sms / get_num_sms. */
dg_status dg_set_num_cus(int num_cus);
int dg_get_num_cus(void);

/* Static text for a status code (never NULL). */
const char* dg_status_string(dg_status s);

/* Text of the last HIP error seen by this thread inside the library ("" if none). */
const char* dg_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DG_H */
