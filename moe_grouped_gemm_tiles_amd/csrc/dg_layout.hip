// dg_layout.hip -- scale-factor layout transform of libdg on gfx950.
//
// Source: DeepGEMM README as mirrored on "Weight gradient kernels for dense
// and MoE models #95", section "Utilities" (transform scaling factors into
// the required layout: MN-major, TMA-aligned, optionally packed into UE8M0)
// and "Interfaces > Notices" (the LHS scale factor is transposed and aligned;
// UE8M0 packs four scale bytes into one 32-bit int).
//
// Per-row scales sf[g][r][kb] (row-major, K blocks contiguous) become the
// GEMM's sfa operand: FP32 out[g][kb][r] with row stride ld, or int32 words
// out[g][q][r] whose byte j is the biased exponent field of sf[g][r][4q+j]
// (exact for powers of two; 127 past the last K block).  A workgroup moves a
// tile of 64 rows x 32 K blocks through LDS so that both the reads (along K)
// and the writes (along rows) are contiguous runs.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "dg.h"
#include "dg_common.hpp"

namespace {

constexpr int kRows = 64, kBlocks = 32, kThreads = 256;

__global__ void __launch_bounds__(kThreads) sf_layout_kernel(const float* sf, int rows, int kb, int64_t in_gs,
                                                             void* out, int64_t ld, int64_t out_gs, int ue8m0) {
  __shared__ float t[kBlocks][kRows + 1];
  const int tid = threadIdx.x;
  const int r0 = blockIdx.x * kRows, k0 = blockIdx.y * kBlocks;
  const float* in = sf + (int64_t)blockIdx.z * in_gs;
  for (int rr = tid / kBlocks; rr < kRows; rr += kThreads / kBlocks) {
    const int r = r0 + rr, k = k0 + tid % kBlocks;
    t[tid % kBlocks][rr] = (r < rows && k < kb) ? in[(int64_t)r * kb + k] : 0.f;
  }
  __syncthreads();
  const int rr = tid % kRows, r = r0 + rr;
  if (r >= rows) return;
  if (!ue8m0) {
    float* o = static_cast<float*>(out) + (int64_t)blockIdx.z * out_gs;
    for (int kk = tid / kRows; kk < kBlocks; kk += kThreads / kRows) {
      const int k = k0 + kk;
      if (k < kb) o[(int64_t)k * ld + r] = t[kk][rr];
    }
  } else {
    int32_t* o = static_cast<int32_t*>(out) + (int64_t)blockIdx.z * out_gs;
    for (int qq = tid / kRows; qq < kBlocks / 4; qq += kThreads / kRows) {
      const int q = k0 / 4 + qq;
      if (4 * q >= kb) continue;
      uint32_t w = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t byte = 4 * q + j < kb ? (__float_as_uint(t[4 * qq + j][rr]) >> 23) & 0xFFu : 127u;
        w |= byte << (8 * j);
      }
      o[(int64_t)q * ld + r] = (int32_t)w;
    }
  }
}

}  // namespace

extern "C" {

dg_status dg_transform_sf_into_required_layout(const float* sf, void* out, int num_groups, int mn, int kb,
                                               int64_t ld_out, int ue8m0, hipStream_t stream) {
  if (num_groups < 0 || mn < 0 || kb < 0) return DG_ERROR_INVALID_VALUE;
  if (num_groups == 0 || mn == 0 || kb == 0) return DG_SUCCESS;
  if (sf == nullptr || out == nullptr) return DG_ERROR_INVALID_VALUE;
  if (reinterpret_cast<uintptr_t>(sf) % 4 != 0 || reinterpret_cast<uintptr_t>(out) % 16 != 0)
    return DG_ERROR_INVALID_VALUE;
  if (ld_out < mn || ld_out % 4 != 0) return DG_ERROR_INVALID_VALUE;
  if (num_groups > 65535) return DG_ERROR_NOT_SUPPORTED;
  const int64_t out_rows = ue8m0 ? (kb + 3) / 4 : kb;
  const dim3 grid((mn + kRows - 1) / kRows, (kb + kBlocks - 1) / kBlocks, num_groups);
  hipLaunchKernelGGL(sf_layout_kernel, grid, dim3(kThreads), 0, stream, sf, mn, kb, (int64_t)mn * kb, out, ld_out,
                     out_rows * ld_out, ue8m0 ? 1 : 0);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? DG_SUCCESS : dg::record_hip_error(e);
}

}  // extern "C"
