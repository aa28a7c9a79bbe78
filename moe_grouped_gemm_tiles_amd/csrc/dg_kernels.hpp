// dg_kernels.hpp -- gfx950 (CDNA4) kernels of libdg: fine-grained-scaled FP8
// GEMM, D = C + A @ B.T, NT layout, dense / M-grouped contiguous / M-grouped
// masked.
//
// Sources (page titles and sections):
//   DeepGEMM README as mirrored on "Weight gradient kernels for dense and MoE
//   models #95": "Interfaces > Notices" (operation, NT layout, FP32 scales,
//   transposed LHS scales), "Grouped GEMMs (contiguous layout)", "Grouped GEMMs
//   (masked layout)".  GeekNews digest "DeepGEMM: बारीक scaling के जरिए साफ़ और
//   efficient FP8 GEMM kernel", Hacker News comments: MMA partial sums are
//   promoted into higher-precision FP32 accumulators with FMAs that should
//   overlap the matrix instructions.
//
// Design (gfx950):
//   * One workgroup owns a BM x BN output tile and walks K in 128-wide slabs;
//     each slab is exactly one scale block along K.
//   * A and B slabs are staged global -> VGPR -> LDS, double buffered (the
//     next slab's global loads are in flight while the current slab is
//     multiplied).  LDS rows are 128 bytes; 16-byte chunks are XOR-swizzled by
//     (row & 7) so that both the 16-byte writes and the 16-byte fragment reads
//     of 8 consecutive rows hit 8 different bank groups.
//   * Each wave owns a (BM/WM) x (BN/WN) sub-tile made of 16x16 MFMA tiles.
//     One v_mfma_f32_16x16x128_f8f6f4 covers a full 128-K slab of a 16x16
//     tile, so the slab partial of a tile is a single instruction with a zero
//     accumulator input.  B is passed as the MFMA's first operand and A as the
//     second, so that a lane's four results are four consecutive columns of
//     one output row: the row scale sfa is then one value per lane per
//     16-row fragment and the stores are 8/16-byte vectors.
//   * Promotion: acc += P * (sfa[row] * sfb[block]) in FP32 after every slab.
//   * Persistent grid: blockIdx strides over the tile list; grouped variants
//     resolve the group on device (contiguous: from the first row's group
//     index; masked: from masked_m), so the host never synchronises.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum Mode : int { MODE_DENSE = 0, MODE_CONTIG = 1, MODE_MASKED = 2 };

// Kernel arguments.  Strides in elements of the pointed-to type.
struct Params {
  const uint8_t* a;
  const float* sfa;
  const uint8_t* b;
  const float* sfb;
  const void* c;
  void* d;
  const int32_t* grp;  // contiguous: m_indices[M]; masked: masked_m[G]
  int64_t lda, ldb, ldc, ldd, ld_sfa;
  int64_t a_gs, sfa_gs, b_gs, sfb_gs, d_gs;  // per-group strides
  int m, n, k, num_groups;
  int tiles_m, tiles_n, num_tiles;
};

// v_mfma_f32_16x16x128_f8f6f4 with both operands in E4M3 (format code 0) and
// no block scaling (zero scale operands select the unscaled instruction).
// Result lane l, element r: row (l % 16) of operand y, column 4*(l/16)+r of
// operand x, i.e. out[x_row = 4*(l/16)+r][y_row = l%16] = sum_k x[.,k]*y[.,k].
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(i32x8 x, i32x8 y) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, zero, 0, 0, 0, 0, 0, 0);
}

// FP32 -> BF16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Grouped raster: GM m-tiles at a time sweep all n-tiles, so concurrently
// running workgroups share A and B panels in L2.
__device__ __forceinline__ void raster(int t, int tm, int tn, int& mb, int& nb) {
  constexpr int GM = 8;
  const int per = GM * tn;
  const int grp = t / per;
  const int first = grp * GM;
  const int gsz = min(tm - first, GM);
  const int r = t - grp * per;
  mb = first + r % gsz;
  nb = r / gsz;
}

template <int BM, int BN, int WM, int WN, int MODE, bool BF16_OUT, bool HAS_C>
__global__ void __launch_bounds__(WM * WN * 64) gemm_kernel(const Params p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int A_CH = BM * 8 / NT, B_CH = BN * 8 / NT;  // 16-byte chunks per thread per slab
  constexpr int STAGE = (BM + BN) * 128;
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be whole 16x16 MFMA tiles");
  static_assert(A_CH * NT == BM * 8 && B_CH * NT == BN * 8, "slab must split evenly over threads");

  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int KB = p.k >> 7;
  const int NBLK = (p.n + 127) >> 7;
  const int tiles_mn = p.tiles_m * p.tiles_n;

  for (int tile = blockIdx.x; tile < p.num_tiles; tile += gridDim.x) {
    int g = 0, t = tile;
    if (MODE == MODE_MASKED) {
      g = t / tiles_mn;
      t -= g * tiles_mn;
    }
    int mb, nb;
    raster(t, p.tiles_m, p.tiles_n, mb, nb);
    const int m0 = mb * BM, n0 = nb * BN;

    int row_end = p.m;  // rows >= row_end are never stored
    if (MODE == MODE_MASKED) {
      const int mm = min(max(p.grp[g], 0), p.m);
      if (m0 >= mm) continue;
      row_end = mm;
    } else if (MODE == MODE_CONTIG) {
      g = p.grp[m0];
      if (g < 0 || g >= p.num_groups) continue;
    }

    const uint8_t* A = p.a + (MODE == MODE_MASKED ? (int64_t)g * p.a_gs : 0);
    const float* SFA = p.sfa + (MODE == MODE_MASKED ? (int64_t)g * p.sfa_gs : 0);
    const uint8_t* B = p.b + (MODE != MODE_DENSE ? (int64_t)g * p.b_gs : 0);
    const float* SFB = p.sfb + (MODE != MODE_DENSE ? (int64_t)g * p.sfb_gs : 0);

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    i32x4 ra[A_CH], rb[B_CH];
    auto gload = [&](int kb) {
#pragma unroll
      for (int i = 0; i < A_CH; ++i) {
        const int c = tid + i * NT, row = c >> 3, ch = c & 7;
        const int gm = m0 + row;
        ra[i] = gm < p.m ? *reinterpret_cast<const i32x4*>(A + (int64_t)gm * p.lda + kb * 128 + ch * 16)
                         : i32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = tid + i * NT, row = c >> 3, ch = c & 7;
        const int gn = n0 + row;
        rb[i] = gn < p.n ? *reinterpret_cast<const i32x4*>(B + (int64_t)gn * p.ldb + kb * 128 + ch * 16)
                         : i32x4{0, 0, 0, 0};
      }
    };
    auto lstore = [&](int buf) {
      uint8_t* base = lds + buf * STAGE;
#pragma unroll
      for (int i = 0; i < A_CH; ++i) {
        const int c = tid + i * NT, row = c >> 3, ch = c & 7;
        *reinterpret_cast<i32x4*>(base + row * 128 + ((ch ^ (row & 7)) << 4)) = ra[i];
      }
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = tid + i * NT, row = c >> 3, ch = c & 7;
        *reinterpret_cast<i32x4*>(base + BM * 128 + row * 128 + ((ch ^ (row & 7)) << 4)) = rb[i];
      }
    };

    if (KB > 0) {
      gload(0);
      lstore(0);
    }
    __syncthreads();

    for (int kb = 0; kb < KB; ++kb) {
      const int cur = kb & 1;
      if (kb + 1 < KB) gload(kb + 1);

      float sa[FM], sb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int gm = m0 + wm * TM + i * 16 + r16;
        sa[i] = gm < p.m ? SFA[(int64_t)kb * p.ld_sfa + gm] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int bn = (n0 + wn * TN + j * 16) >> 7;
        sb[j] = bn < NBLK ? SFB[(int64_t)bn * KB + kb] : 0.f;
      }

      const uint8_t* As = lds + cur * STAGE;
      const uint8_t* Bs = As + BM * 128;
      const int sw0 = ((2 * q4) ^ (r16 & 7)) << 4;
      const int sw1 = ((2 * q4 + 1) ^ (r16 & 7)) << 4;
      i32x8 fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint8_t* rowp = As + (wm * TM + i * 16 + r16) * 128;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(rowp + sw0);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(rowp + sw1);
        fa[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint8_t* rowp = Bs + (wn * TN + j * 16 + r16) * 128;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(rowp + sw0);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(rowp + sw1);
        fb[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const f32x4 part = mfma_fp8_16x16x128(fb[j], fa[i]);
          const float s = sa[i] * sb[j];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(part[r], s, acc[i][j][r]);
        }

      if (kb + 1 < KB) lstore(cur ^ 1);
      __syncthreads();
    }

    // Epilogue: D = C + acc, masked stores.
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int gm = m0 + wm * TM + i * 16 + r16;
      bool row_ok = gm < row_end;
      if (MODE == MODE_CONTIG) row_ok = row_ok && p.grp[gm] == g;
      if (!row_ok) continue;
      const int64_t drow = (MODE == MODE_MASKED ? (int64_t)g * p.d_gs : 0) + (int64_t)gm * p.ldd;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int gn = n0 + wn * TN + j * 16 + 4 * q4;
        if (gn >= p.n) continue;
        f32x4 v = acc[i][j];
        const bool full = gn + 4 <= p.n;
        if (HAS_C) {
          const int64_t crow = (int64_t)gm * p.ldc;
          if (BF16_OUT) {
            const uint16_t* C = reinterpret_cast<const uint16_t*>(p.c) + crow + gn;
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (full || gn + r < p.n) v[r] += __uint_as_float((uint32_t)C[r] << 16);
          } else {
            const float* C = reinterpret_cast<const float*>(p.c) + crow + gn;
            if (full) {
              const f32x4 cv = *reinterpret_cast<const f32x4*>(C);
              v += cv;
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (gn + r < p.n) v[r] += C[r];
            }
          }
        }
        if (BF16_OUT) {
          uint16_t* D = reinterpret_cast<uint16_t*>(p.d) + drow + gn;
          if (full) {
            const uint32_t lo = bf16_rne_bits(v[0]) | (bf16_rne_bits(v[1]) << 16);
            const uint32_t hi = bf16_rne_bits(v[2]) | (bf16_rne_bits(v[3]) << 16);
            *reinterpret_cast<uint2*>(D) = make_uint2(lo, hi);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (gn + r < p.n) D[r] = (uint16_t)bf16_rne_bits(v[r]);
          }
        } else {
          float* D = reinterpret_cast<float*>(p.d) + drow + gn;
          if (full) {
            *reinterpret_cast<f32x4*>(D) = v;
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (gn + r < p.n) D[r] = v[r];
          }
        }
      }
    }
    __syncthreads();  // LDS of this tile is free before the next tile's first stores
  }
}

}  // namespace dg
