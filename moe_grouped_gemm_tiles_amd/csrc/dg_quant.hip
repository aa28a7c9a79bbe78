// dg_quant.hip -- FP8 (E4M3) quantization of GEMM operands on gfx950: the
// cast the GEMM's caller performs, fused into one pass that also writes the
// scale factors in the layout the GEMM entry points take.
//
// Source: DeepGEMM README as mirrored on "Weight gradient kernels for dense
// and MoE models #95", section "Interfaces > Notices" (FP8 casting is the
// caller's job; the LHS scale factors must be transposed and aligned; FP32
// scales on one architecture, UE8M0 packed four per int on the other) and
// section "Utilities" (helpers that put scale factors into that layout).
// Readings (the pages give no block shape or scale rule):
//   * per-token: one scale per (row, 128 consecutive K elements), written
//     transposed, sf[kb][m] (FP32) or sf[kb/4][m] (four UE8M0 bytes per word);
//   * per-block: one scale per 128 x 128 block, sf[nb][kb] (FP32) or
//     sf[nb][kb/4] (packed UE8M0);
//   * FP32 scale s = amax / 448 in FP32 (448 = E4M3's largest finite value),
//     s = 1 for an all-zero block; UE8M0 scale = the smallest power of two
//     2^e >= fp32(amax / 448) (1 for an all-zero block), byte e + 127;
//   * code = E4M3(clamp(x / s, -448, 448)), the quotient rounded to FP32
//     (a correctly rounded division), then to E4M3 with ties to even.
//
// Both kernels are HBM-bound (read 2 or 4 bytes, write 1 byte per element):
//   * per-token: a workgroup owns 64 rows x 512 columns; each 16-lane group
//     reads one (row, 128-block) as 16-byte vectors (the four blocks of a row
//     are contiguous, so a wave reads 1 KiB runs), reduces amax across its 16
//     lanes, and writes 8 code bytes per lane.  The workgroup's 4 x 64 scales
//     go through LDS and leave as 256-byte runs of the transposed layout (or
//     as 64 packed UE8M0 words).
//   * per-block: a workgroup owns one 128 x 128 block, holds it in registers
//     (64 values per lane) between the amax reduction and the quantization.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "dg.h"
#include "dg_common.hpp"

namespace {

namespace q {

constexpr float kE4M3Max = 448.0f;

// FP32 scale of a block with the given amax.
__device__ __forceinline__ float fp32_scale(float amax) { return amax == 0.0f ? 1.0f : amax / kE4M3Max; }

// UE8M0 exponent byte of the smallest power of two >= fp32(amax / 448).
__device__ __forceinline__ uint32_t ue8m0_byte(float amax) {
  if (amax == 0.0f) return 127u;
  const float t = amax / kE4M3Max;
  int ex;
  const float mant = frexpf(t, &ex);  // t = mant * 2^ex, mant in [0.5, 1)
  int e = (mant == 0.5f) ? ex - 1 : ex;
  e += 127;
  return (uint32_t)(e < 0 ? 0 : (e > 254 ? 254 : e));
}

// 2^(byte - 127) as FP32 (denormal for byte 0).
__device__ __forceinline__ float ue8m0_value(uint32_t byte) { return ldexpf(1.0f, (int)byte - 127); }

// Four FP32 values -> four E4M3 bytes (hardware conversion, round to nearest
// even), after clamping to the finite range.
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -kE4M3Max), kE4M3Max);
  b = fminf(fmaxf(b, -kE4M3Max), kE4M3Max);
  c = fminf(fmaxf(c, -kE4M3Max), kE4M3Max);
  d = fminf(fmaxf(d, -kE4M3Max), kE4M3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Eight input values starting at p (16 bytes of BF16 or 32 bytes of FP32).
template <bool BF16_IN>
__device__ __forceinline__ void load8(const void* p, float v[8]) {
  if constexpr (BF16_IN) {
    const uint4 r = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float4 lo = *reinterpret_cast<const float4*>(p);
    const float4 hi = *(reinterpret_cast<const float4*>(p) + 1);
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  }
}

// The correctly rounded FP32 division x / s is the fused multiply-add sequence
// of the IEEE division (reciprocal estimate, one refinement, quotient, two
// corrections), wrapped in range scaling that only acts when the divisor is
// denormal or above 2^126, the quotient is denormal, the numerator is below
// 2^-104 or the operands' exponents are 96 or more apart.  For a divisor in
// [2^-80, 2^100] and |x| <= 448 s (x from the divisor's own block) none of
// that applies to a quotient of 2^-10 or more, so there the bare sequence gives
// the same quotient, and its reciprocal part -- which depends on s alone -- is
// done once for the eight values.  Smaller quotients round to an E4M3 zero
// either way; the sign of x is put back so that -0 and negative underflows
// still give the negative zero code.
__device__ __forceinline__ bool plain_div_range(float s) { return s >= 0x1p-80f && s <= 0x1p100f; }
__device__ __forceinline__ float refined_recip(float s) {
  const float r = __builtin_amdgcn_rcpf(s);
  return __builtin_fmaf(__builtin_fmaf(-s, r, 1.0f), r, r);
}
__device__ __forceinline__ float div_by(float x, float s, float y) {
  const float q0 = x * y;
  const float q1 = __builtin_fmaf(__builtin_fmaf(-s, q0, x), y, q0);
  const float q2 = __builtin_fmaf(__builtin_fmaf(-s, q1, x), y, q1);
  return __builtin_copysignf(q2, x);
}

// Quantize eight values with scale s (FP32 path: correctly rounded x / s).
template <bool UE8M0>
__device__ __forceinline__ uint2 quant8(const float v[8], float s) {
  float y[8];
  if (UE8M0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = v[i] * (1.0f / s);  // 1/s is exact for a power of two
  } else if (plain_div_range(s)) {
    const float r = refined_recip(s);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = div_by(v[i], s, r);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = v[i] / s;
  }
  return make_uint2(pack4(y[0], y[1], y[2], y[3]), pack4(y[4], y[5], y[6], y[7]));
}

constexpr int kTokRows = 64;   // rows per workgroup
constexpr int kTokBlocks = 4;  // 128-K blocks per workgroup (one packed UE8M0 word)

template <bool BF16_IN, bool UE8M0>
__global__ void __launch_bounds__(256) per_token_kernel(const uint8_t* __restrict__ x, int64_t ldx_bytes,
                                                        uint8_t* __restrict__ qo, int64_t ldq, void* __restrict__ sf,
                                                        int64_t ld_sf, int m, int k) {
  __shared__ float s_blk[kTokBlocks][kTokRows];  // FP32 scale or UE8M0 byte (as float) per block
  constexpr int ES = BF16_IN ? 2 : 4;
  const int tid = threadIdx.x, grp = tid >> 4, l = tid & 15;
  const int m0 = blockIdx.x * kTokRows;
  const int kb0 = blockIdx.y * kTokBlocks;
  const int nkb = min(kTokBlocks, (k >> 7) - kb0);
  for (int b = grp; b < kTokRows * kTokBlocks; b += 16) {
    const int r = b >> 2, j = b & 3;  // the four blocks of a row are adjacent: 1 KiB (BF16) runs
    const int row = m0 + r;
    if (row >= m || j >= nkb) continue;  // uniform across the 16-lane group
    const int col = (kb0 + j) * 128 + 8 * l;
    float v[8];
    load8<BF16_IN>(x + (int64_t)row * ldx_bytes + (int64_t)col * ES, v);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
    float s;
    if constexpr (UE8M0) {
      const uint32_t e = ue8m0_byte(amax);
      s = ue8m0_value(e);
      if (l == 0) s_blk[j][r] = (float)e;
    } else {
      s = fp32_scale(amax);
      if (l == 0) s_blk[j][r] = s;
    }
    *reinterpret_cast<uint2*>(qo + (int64_t)row * ldq + col) = quant8<UE8M0>(v, s);
  }
  __syncthreads();
  if constexpr (UE8M0) {
    if (tid < kTokRows && m0 + tid < m) {
      uint32_t w = 0;
#pragma unroll
      for (int j = 0; j < kTokBlocks; ++j) w |= (j < nkb ? (uint32_t)s_blk[j][tid] : 127u) << (8 * j);
      reinterpret_cast<uint32_t*>(sf)[(int64_t)blockIdx.y * ld_sf + m0 + tid] = w;
    }
  } else {
    for (int idx = tid; idx < nkb * kTokRows; idx += 256) {
      const int j = idx / kTokRows, r = idx % kTokRows;
      if (m0 + r < m) reinterpret_cast<float*>(sf)[(int64_t)(kb0 + j) * ld_sf + m0 + r] = s_blk[j][r];
    }
  }
}

// (held to 96 registers, five waves per SIMD: the division's per-block reciprocal
// would otherwise tip the FP32-scale variant to four)
template <bool BF16_IN, bool UE8M0>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5)))
per_block_kernel(const uint8_t* __restrict__ w, int64_t ldw_bytes, uint8_t* __restrict__ qo, int64_t ldq,
                 void* __restrict__ sf, int n, int k) {
  __shared__ float s_amax[4];
  constexpr int ES = BF16_IN ? 2 : 4;
  const int tid = threadIdx.x, rg = tid >> 4, l = tid & 15;
  const int kb = blockIdx.x, nb = blockIdx.y;
  const int KB = k >> 7;
  const int col = kb * 128 + 8 * l;
  float v[8][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = nb * 128 + rg + 16 * i;
    if (row < n) {
      load8<BF16_IN>(w + (int64_t)row * ldw_bytes + (int64_t)col * ES, v[i]);
#pragma unroll
      for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(v[i][c]));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((tid & 63) == 0) s_amax[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_amax[0], s_amax[1]), fmaxf(s_amax[2], s_amax[3]));
  float s;
  uint32_t e = 0;
  if constexpr (UE8M0) {
    e = ue8m0_byte(amax);
    s = ue8m0_value(e);
  } else {
    s = fp32_scale(amax);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = nb * 128 + rg + 16 * i;
    if (row < n) *reinterpret_cast<uint2*>(qo + (int64_t)row * ldq + col) = quant8<UE8M0>(v[i], s);
  }
  if (tid == 0) {
    if constexpr (UE8M0) {
      // bytes of a packed word belong to four workgroups; each writes its own,
      // and the one with the last K block also writes the padding bytes (127)
      const int kq = (KB + 3) >> 2;
      uint8_t* bytes = reinterpret_cast<uint8_t*>(sf) + ((int64_t)nb * kq + (kb >> 2)) * 4;
      bytes[kb & 3] = (uint8_t)e;
      if (kb == KB - 1)
        for (int j = (kb & 3) + 1; j < 4; ++j) bytes[j] = 127;
    } else {
      reinterpret_cast<float*>(sf)[(int64_t)nb * KB + kb] = s;
    }
  }
}

}  // namespace q

dg_status quant_launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? DG_SUCCESS : dg::record_hip_error(e);
}

inline bool aligned_to(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

}  // namespace

extern "C" {

dg_status dg_per_token_cast_to_fp8(const void* x, int64_t ldx, dg_dtype x_dtype, void* q, int64_t ldq, void* sf,
                                   int64_t ld_sf, int ue8m0, int m, int k, hipStream_t stream) {
  if (m < 0 || k < 0 || (x_dtype != DG_DTYPE_BF16 && x_dtype != DG_DTYPE_FP32)) return DG_ERROR_INVALID_VALUE;
  if (k % 128 != 0) return DG_ERROR_NOT_SUPPORTED;
  if (m == 0 || k == 0) return DG_SUCCESS;
  const int64_t es = x_dtype == DG_DTYPE_BF16 ? 2 : 4;
  if (x == nullptr || q == nullptr || sf == nullptr) return DG_ERROR_INVALID_VALUE;
  if (!aligned_to(x, 16) || !aligned_to(q, 8) || !aligned_to(sf, 16)) return DG_ERROR_INVALID_VALUE;
  if (ldx < k || (ldx * es) % 16 != 0 || ldq < k || ldq % 8 != 0) return DG_ERROR_INVALID_VALUE;
  if (ld_sf < m || ld_sf % 4 != 0) return DG_ERROR_INVALID_VALUE;
  const dim3 grid((m + q::kTokRows - 1) / q::kTokRows, (k / 128 + q::kTokBlocks - 1) / q::kTokBlocks);
  if (grid.y > 65535) return DG_ERROR_NOT_SUPPORTED;
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  uint8_t* qb = static_cast<uint8_t*>(q);
  const int64_t ldx_b = ldx * es;
  if (x_dtype == DG_DTYPE_BF16) {
    if (ue8m0) hipLaunchKernelGGL((q::per_token_kernel<true, true>), grid, dim3(256), 0, stream, xb, ldx_b, qb, ldq, sf, ld_sf, m, k);
    else hipLaunchKernelGGL((q::per_token_kernel<true, false>), grid, dim3(256), 0, stream, xb, ldx_b, qb, ldq, sf, ld_sf, m, k);
  } else {
    if (ue8m0) hipLaunchKernelGGL((q::per_token_kernel<false, true>), grid, dim3(256), 0, stream, xb, ldx_b, qb, ldq, sf, ld_sf, m, k);
    else hipLaunchKernelGGL((q::per_token_kernel<false, false>), grid, dim3(256), 0, stream, xb, ldx_b, qb, ldq, sf, ld_sf, m, k);
  }
  return quant_launch_status();
}

dg_status dg_per_block_cast_to_fp8(const void* w, int64_t ldw, dg_dtype w_dtype, void* q, int64_t ldq, void* sf,
                                   int ue8m0, int n, int k, hipStream_t stream) {
  if (n < 0 || k < 0 || (w_dtype != DG_DTYPE_BF16 && w_dtype != DG_DTYPE_FP32)) return DG_ERROR_INVALID_VALUE;
  if (k % 128 != 0) return DG_ERROR_NOT_SUPPORTED;
  if (n == 0 || k == 0) return DG_SUCCESS;
  const int64_t es = w_dtype == DG_DTYPE_BF16 ? 2 : 4;
  if (w == nullptr || q == nullptr || sf == nullptr) return DG_ERROR_INVALID_VALUE;
  if (!aligned_to(w, 16) || !aligned_to(q, 8) || !aligned_to(sf, 4)) return DG_ERROR_INVALID_VALUE;
  if (ldw < k || (ldw * es) % 16 != 0 || ldq < k || ldq % 8 != 0) return DG_ERROR_INVALID_VALUE;
  const dim3 grid(k / 128, (n + 127) / 128);
  if (grid.y > 65535) return DG_ERROR_NOT_SUPPORTED;
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  uint8_t* qb = static_cast<uint8_t*>(q);
  const int64_t ldw_b = ldw * es;
  if (w_dtype == DG_DTYPE_BF16) {
    if (ue8m0) hipLaunchKernelGGL((q::per_block_kernel<true, true>), grid, dim3(256), 0, stream, wb, ldw_b, qb, ldq, sf, n, k);
    else hipLaunchKernelGGL((q::per_block_kernel<true, false>), grid, dim3(256), 0, stream, wb, ldw_b, qb, ldq, sf, n, k);
  } else {
    if (ue8m0) hipLaunchKernelGGL((q::per_block_kernel<false, true>), grid, dim3(256), 0, stream, wb, ldw_b, qb, ldq, sf, n, k);
    else hipLaunchKernelGGL((q::per_block_kernel<false, false>), grid, dim3(256), 0, stream, wb, ldw_b, qb, ldq, sf, n, k);
  }
  return quant_launch_status();
}

}  // extern "C"
