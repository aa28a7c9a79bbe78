// dg_mqa.hip -- weighted-ReLU MQA logits (the lightning-indexer scoring
// kernel) on gfx950.
//
// Source: DeepGEMM README as mirrored on "Weight gradient kernels for dense
// and MoE models #95", section "V3.2 MQA kernels for the indexer": for query
// i and every key j in [ks[i], ke[i]),
//     out[i, j] = sum_h w[i, h] * relu( q[i, h, :] . (kv[j, :] * sf[j]) )
// with q E4M3 [S, H, D], kv E4M3 [S_kv, D] with one FP32 scale per row,
// w FP32 [S, H]; positions outside the range are set to -inf when
// clean_logits is set.  Readings: logits are FP32; ks/ke are clamped to
// [0, S_kv]; without clean_logits the positions outside the range are left
// untouched; the kv scales are non-negative (they are quantization scales),
// so relu(sf * x) = sf * relu(x) and sf is applied once per key after the
// head sum.
//
// Mapping: head_dim D = 128 is exactly one K slab of v_mfma_f32_16x16x128_f8f6f4,
// so one MFMA gives the dot products of 16 heads of one query with 16 keys.
//   * A workgroup (4 waves) owns a tile of 256 keys and 32 queries.  The kv
//     tile (32 KiB) is staged once in LDS with direct global->LDS loads, rows
//     XOR-swizzled like the GEMM's.  Every query re-reads its q rows from
//     global memory once per key tile, so the wider the tile the less q
//     traffic; 256 keys keep the kernel at three waves per SIMD.
//   * Each wave streams its 8 queries: 4 head fragments of q straight from
//     global memory (the next query's are loaded while the current one is
//     computed), then key fragment by key fragment (read from LDS one
//     fragment ahead) 4 MFMAs, one per head fragment, and per MFMA output
//     value one integer max (the ReLU) and one FMA with the head weight,
//     issued three MFMAs behind.  q is the MFMA's first operand, so a lane
//     holds four heads of one key and the head sum is four FMAs per lane plus
//     two lane swaps (v_permlane32_swap, v_permlane16_swap) and adds per key.
//   * Two FP32 VALU operations per (query, head, key) against 256 MFMA flops
//     put the VALU and the matrix core at about the same peak rate on this
//     chip, so the kernel is bound by both once q traffic is amortised.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "dg.h"
#include "dg_common.hpp"

namespace {

namespace mqa {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kKeys = 256;     // keys per workgroup tile
constexpr int kHalves = kKeys / 128;  // 8 key fragments per head-sum scatter
constexpr int kQueries = 32;   // queries per workgroup
constexpr int kWaves = 4;
constexpr int kD = 128;        // head dim = one MFMA K slab
constexpr int kMaxHeads = 64;

struct Params {
  const uint8_t* q;
  const uint8_t* kv;
  const float* sf;
  const float* w;
  const int32_t* ks;
  const int32_t* ke;
  float* out;
  int64_t ld_out;
  int s, s_kv, h;
  int clean;
};

// Head sum of 8 per-key-fragment partial sums of a lane (one 128-key half of
// the tile) across the four lane groups (each group holds 4 of every 16
// heads), scattered so that lane group g ends with the sums of key fragments
// 2g and 2g+1 of that half -- the two it stores.
// v_permlane32_swap(a, b) returns ([a_lo, b_lo], [a_hi, b_hi]) by 32-lane
// halves and v_permlane16_swap the same by 16-lane rows (checked on gfx950),
// so one swap and one add fold two values at once; six swaps and six adds in
// all, on the VALU (no trip through the LDS unit as __shfl_xor takes).
__device__ __forceinline__ void head_sum_scatter(const float (&acc)[8], float (&out)[2]) {
  float r[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[k]), __float_as_uint(acc[k + 4]), false, false);
    r[k] = __uint_as_float(a[0]) + __uint_as_float(a[1]);  // halves: key k (lanes 0-31), key k+4 (32-63)
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(r[k]), __float_as_uint(r[k + 2]), false, false);
    out[k] = __uint_as_float(b[0]) + __uint_as_float(b[1]);  // rows: keys k, k+2, k+4, k+6
  }
}

// max(x, 0) for a float as one integer max on its bits: negative values
// (sign bit set) become +0, everything else is kept.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Wave-uniform load through the scalar cache: a uniform address in the
// constant address space makes the compiler emit s_load (counted by lgkmcnt
// only; a flat load would also occupy the vector-load counter and make the
// value a per-lane one).  The ranges are read-only during the kernel.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
__device__ __forceinline__ int load_uniform_i32(const int32_t* ptr) {
  const uint64_t a = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return *reinterpret_cast<const_i32_ptr>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ f32x4 mfma(i32x8 x, i32x8 y) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, zero, 0, 0, 0, 0, 0, 0);
}

template <int H>
__global__ void __launch_bounds__(kWaves * 64) logits_kernel(const Params p) {
  constexpr int HT = H / 16;  // 16-head fragments per query
  __shared__ __attribute__((aligned(1024))) uint8_t kv_lds[kKeys * kD];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, q4 = lane >> 4;
  // Workgroups go to the 8 XCDs round-robin in launch order (x fastest).  When
  // the query blocks come in multiples of 8, XCD x takes query blocks x, x + 8,
  // ... with all their key tiles in a row, so a block's q rows are fetched into
  // one XCD's L2 instead of all eight, and the causal work stays spread evenly.
  int kt_idx = blockIdx.x, qb_idx = blockIdx.y;
  if ((gridDim.y & 7) == 0) {
    const int lin = blockIdx.y * gridDim.x + blockIdx.x;
    const int xcd = lin & 7, slot = lin >> 3;
    qb_idx = xcd + 8 * (slot / (int)gridDim.x);
    kt_idx = slot % (int)gridDim.x;
  }
  const int key0 = kt_idx * kKeys;
  const int qry0 = qb_idx * kQueries;

  // Does any query of this workgroup see a key of this tile?
  bool any = false;
  for (int i = qry0 + (tid & 31); i < min(qry0 + kQueries, p.s) && tid < 32; i += 32) {
    const int lo = min(max(p.ks[i], 0), p.s_kv), hi = min(max(p.ke[i], 0), p.s_kv);
    any = any || (lo < hi && lo < key0 + kKeys && hi > key0);
  }
  any = __syncthreads_or(any);

  if (any) {
    // kv tile -> LDS: 16 direct 1 KiB loads, 4 per wave; row r's 16-byte chunk
    // c lands at chunk c ^ (r & 7) (the global address is permuted instead).
    const int ld_row = lane >> 3, ld_chunk = ((lane & 7) ^ (lane >> 3)) << 4;
    const int64_t rows_left = (int64_t)p.s_kv - key0;
    const uint32_t bytes = rows_left <= 0 ? 0u : (uint32_t)min<int64_t>(rows_left * kD, 0x7fffffff);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.kv + (int64_t)key0 * kD), (short)0, (int)bytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < kKeys * kD / 1024 / kWaves; ++i) {
      const int blk = wave * (kKeys * kD / 1024 / kWaves) + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(kv_lds + blk * 1024), 16,
                                               (uint32_t)((blk * 8 + ld_row) * kD + ld_chunk), 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt((0) | (0x7 << 4) | (0xF << 8));  // vmcnt(0)
    __syncthreads();
  }
  // key fragment kt of the tile from LDS (lane: key kt*16 + r16, K chunks q4 and q4 + 4)
  const int sw0 = (q4 ^ (r16 & 7)) << 4, sw1 = ((q4 + 4) ^ (r16 & 7)) << 4;
  auto read_kv = [&](int kt) {
    const uint8_t* row = kv_lds + (kt * 16 + r16) * kD;
    const i32x4 lo = *reinterpret_cast<const i32x4*>(row + sw0);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(row + sw1);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };

  // in each 128-key half this lane stores the keys of fragments 2*q4 and 2*q4+1; their scales
  float sfl[2 * kHalves];
#pragma unroll
  for (int u = 0; u < 2 * kHalves; ++u) {
    const int key = key0 + (u >> 1) * 128 + (2 * q4 + (u & 1)) * 16 + r16;
    sfl[u] = key < p.s_kv ? p.sf[key] : 0.f;
  }

  // Operands of query i: q fragment t (lane holds head 16t + r16, K chunks q4
  // and q4 + 4) and the lane's head weights (heads 16t + 4*q4 + r).  Both are
  // loaded one query ahead; loading the weights just before use would make
  // their wait (vector loads complete in order) also wait for the prefetch.
  auto load_q = [&](int i, i32x8 (&f)[HT], f32x4 (&wt)[HT]) {
#pragma unroll
    for (int t = 0; t < HT; ++t) {
      const uint8_t* row = p.q + ((int64_t)i * H + t * 16 + r16) * kD;
      const i32x4 lo = *reinterpret_cast<const i32x4*>(row + 16 * q4);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(row + 64 + 16 * q4);
      f[t] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      wt[t] = *reinterpret_cast<const f32x4*>(p.w + (int64_t)i * H + t * 16 + 4 * q4);
    }
  };

  const int per_wave = kQueries / kWaves;
  static_assert(kQueries % (2 * kWaves) == 0, "queries come in pairs per wave");
  i32x8 qa[HT], qb[HT];
  f32x4 wa[HT], wb[HT];

  // One query: uses (qc, wc), prefetches query i + kWaves into (qn, wn).  The
  // prefetch is unconditional (the index is clamped to a valid query): with a
  // path that skips it, the loop's join would have to wait for every load in
  // flight, the prefetch included.
  auto one_query = [&](int n, i32x8 (&qc)[HT], f32x4 (&wc)[HT], i32x8 (&qn)[HT], f32x4 (&wn)[HT])
                       __attribute__((always_inline)) {
    const int i = qry0 + wave + n * kWaves;
    if (i >= p.s) return;  // wave-uniform
    const int lo = min(max(load_uniform_i32(p.ks + i), 0), p.s_kv);
    const int hi = min(max(load_uniform_i32(p.ke + i), 0), p.s_kv);
    const bool live = any && lo < hi && lo < key0 + kKeys && hi > key0;
    load_q(min(i + kWaves, p.s - 1), qn, wn);
    float sums[2 * kHalves] = {};
    if (live) {
      float acc[kKeys / 16];
#pragma unroll
      for (int kt = 0; kt < kKeys / 16; ++kt) acc[kt] = 0.f;
      // Flat sequence of the HT * (kKeys / 16) MFMAs (key fragment kt = s / HT,
      // head fragment t = s % HT): each key fragment is read from LDS once per
      // query, one fragment ahead, into two register sets.  The ReLU and
      // weight FMAs of MFMA s - (RING - 1) are issued after MFMA s, so they
      // run under the matrix core; every acc[kt] still takes its heads in
      // the order t = 0, 1, ...
      constexpr int T = HT * (kKeys / 16);
      constexpr int RING = 4;
      f32x4 part[RING];
      i32x8 kf[2];
      kf[0] = read_kv(0);
#pragma unroll
      for (int st = 0; st < T + RING - 1; ++st) {
        if (st < T) {
          const int kt = st / HT, t = st % HT;
          if (t == 0 && kt + 1 < kKeys / 16) kf[(kt + 1) & 1] = read_kv(kt + 1);
          part[st % RING] = mfma(qc[t], kf[kt & 1]);
        }
        const int v = st - (RING - 1);
        if (v >= 0) {
          const int kt = v / HT, t = v % HT;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[kt] = __builtin_fmaf(relu(part[v % RING][r]), wc[t][r], acc[kt]);
        }
      }
#pragma unroll
      for (int h = 0; h < kHalves; ++h) {
        float a8[8], s2[2];
#pragma unroll
        for (int k = 0; k < 8; ++k) a8[k] = acc[8 * h + k];
        head_sum_scatter(a8, s2);
        sums[2 * h] = s2[0];
        sums[2 * h + 1] = s2[1];
      }
    }
    if (!live && !p.clean) return;
    float* orow = p.out + (int64_t)i * p.ld_out;
#pragma unroll
    for (int u = 0; u < 2 * kHalves; ++u) {
      const int key = key0 + (u >> 1) * 128 + (2 * q4 + (u & 1)) * 16 + r16;
      if (key >= p.s_kv) continue;
      if (live && key >= lo && key < hi) {
        orow[key] = sums[u] * sfl[u];
      } else if (p.clean) {
        orow[key] = -__builtin_inff();
      }
    }
  };

  load_q(min(qry0 + wave, p.s - 1), qa, wa);
  for (int n = 0; n < per_wave; n += 2) {
    one_query(n, qa, wa, qb, wb);
    one_query(n + 1, qb, wb, qa, wa);
  }
}

}  // namespace mqa

inline bool aligned_to(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

}  // namespace

extern "C" {

dg_status dg_fp8_mqa_logits(const void* q, const void* kv, const float* kv_sf, const float* weights,
                            const int32_t* ks, const int32_t* ke, float* out, int64_t ld_out, int s, int s_kv,
                            int num_heads, int head_dim, int clean_logits, hipStream_t stream) {
  if (s < 0 || s_kv < 0 || num_heads < 0 || head_dim < 0) return DG_ERROR_INVALID_VALUE;
  if (head_dim != mqa::kD || num_heads % 16 != 0 || num_heads > mqa::kMaxHeads || num_heads == 0)
    return DG_ERROR_NOT_SUPPORTED;
  if (s == 0 || s_kv == 0) return DG_SUCCESS;
  if (q == nullptr || kv == nullptr || kv_sf == nullptr || weights == nullptr || ks == nullptr || ke == nullptr ||
      out == nullptr)
    return DG_ERROR_INVALID_VALUE;
  if (!aligned_to(q, 16) || !aligned_to(kv, 16) || !aligned_to(weights, 16) || !aligned_to(kv_sf, 4) ||
      !aligned_to(ks, 4) || !aligned_to(ke, 4) || !aligned_to(out, 4))
    return DG_ERROR_INVALID_VALUE;
  if (ld_out < s_kv) return DG_ERROR_INVALID_VALUE;
  if ((int64_t)s_kv * mqa::kD >= (1ll << 31)) return DG_ERROR_NOT_SUPPORTED;
  const dim3 grid((s_kv + mqa::kKeys - 1) / mqa::kKeys, (s + mqa::kQueries - 1) / mqa::kQueries);
  if (grid.y > 65535) return DG_ERROR_NOT_SUPPORTED;
  mqa::Params p{static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(kv), kv_sf, weights, ks, ke, out,
                ld_out, s, s_kv, num_heads, clean_logits != 0};
  switch (num_heads) {
    case 16: hipLaunchKernelGGL(mqa::logits_kernel<16>, grid, dim3(mqa::kWaves * 64), 0, stream, p); break;
    case 32: hipLaunchKernelGGL(mqa::logits_kernel<32>, grid, dim3(mqa::kWaves * 64), 0, stream, p); break;
    case 48: hipLaunchKernelGGL(mqa::logits_kernel<48>, grid, dim3(mqa::kWaves * 64), 0, stream, p); break;
    default: hipLaunchKernelGGL(mqa::logits_kernel<64>, grid, dim3(mqa::kWaves * 64), 0, stream, p); break;
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? DG_SUCCESS : dg::record_hip_error(e);
}

}  // extern "C"

