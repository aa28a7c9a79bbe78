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
// Design (gfx950; measured: FP8 MFMA ~4.0-4.6 PFLOP/s sustained depending on
// clock, LDS b128 reads ~157 B/clk/CU, direct global->LDS loads ~60 B/clk/CU):
//   * A workgroup owns a BM x BN output tile and walks K in 128-wide slabs;
//     each slab is exactly one scale block along K.
//   * Staging: buffer_load_dwordx4 ... lds copies each slab of A and B (and
//     the slab's BM row scales of A) straight from global memory into LDS,
//     through a ring of STAGES slab buffers, so later slabs stream in while
//     the current one is multiplied.  The buffer descriptors end at the last
//     valid row, so rows past M or N read as zero without any bounds
//     arithmetic.  LDS rows are 128 bytes; 16-byte chunk c of row r sits at
//     chunk c ^ (r & 7), which the loads realise by permuting the global
//     addresses (a direct load writes lane i's 16 bytes at LDS offset 16*i).
//     The 16 lanes of one fragment row group read K chunks q and q+4
//     (q = lane / 16), which together with the swizzle is free of bank
//     conflicts (measured with SQ_LDS_BANK_CONFLICT; the more obvious chunks
//     2q, 2q+1 conflict 2-way on gfx950).
//   * Each wave owns a TM x TN sub-tile of 16x16 MFMA tiles.  One
//     v_mfma_f32_16x16x128_f8f6f4 covers a whole 128-K slab of a 16x16 tile.
//     B is the MFMA's first operand and A the second: a lane's four results
//     are four consecutive columns of one output row, so the row scale is one
//     value per lane per 16-row fragment and stores are 8/16-byte vectors.
//   * FP32 scales: each slab's partial comes out of the MFMA with a zero
//     accumulator and is promoted, acc += P * (sfa[row] * sfb[block]), with
//     FP32 FMAs.  The FMAs of MFMA t are issued after MFMA t+3 (a ring of four
//     partials), so the promotion runs under the matrix core.
//   * UE8M0 scales (powers of two): the MFMA's own block-scale operands apply
//     sfa (per lane = per A row) and sfb (uniform per wave) to every 32-K
//     chunk of the slab, and the MFMA accumulates straight into acc: no
//     promotion at all.
//   * Persistent grid, XCD-aware: workgroup b runs on XCD b % 8, so tile ids
//     are renumbered so that the workgroups of one XCD take consecutive ids,
//     and consecutive ids form compact (GM x n) blocks of tiles that share A
//     and B panels in that XCD's L2.
//   * Grouped variants resolve groups on device (contiguous: group index of a
//     tile's 128-row halves; masked: masked_m; K-grouped: prefix sums of the
//     group K sizes), so the host never synchronises.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

enum Mode : int { MODE_DENSE = 0, MODE_CONTIG = 1, MODE_MASKED = 2, MODE_KGROUP = 3 };

// Kernel arguments.  Strides in elements of the pointed-to type.
struct Params {
  const uint8_t* a;
  const float* sfa;
  const uint8_t* b;
  const float* sfb;
  const void* c;
  void* d;
  const int32_t* grp;  // contiguous: m_indices[M]; masked: masked_m[G]; K-grouped: ks[G]
  int64_t lda, ldb, ldc, ldd, ld_sfa;
  int64_t a_gs, sfa_gs, b_gs, sfb_gs, c_gs, d_gs;  // per-group strides
  int m, n, k, num_groups;
  int tiles_m, tiles_n, num_tiles;
  // split-K (dense only): K slabs are divided into `splits` ranges of
  // `slabs_per_split`, one work unit each.  Every unit writes its FP32
  // partial tile to ws (unit (split s, tile t) at ws + (s * tiles + t) * BM * BN,
  // in fragment order) and counts itself in ctr[t]; the unit that brings the
  // count to `splits` adds the partials in split order, writes D and resets
  // ctr[t] to zero.  ctr must be zero when the kernel starts.
  int splits, slabs_per_split;
  float* ws;
  uint32_t* ctr;
};

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier of the staging ring.  The caller has already waited for
// its own loads of the slab about to be read (vmcnt); this adds the wait for
// the wave's own LDS reads (a stage is overwritten only after every wave has
// read it) and the barrier, but not the vmcnt(0) of __syncthreads(), which
// would drain the loads of later slabs still in flight.  The empty asm
// statements keep the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));  // lgkmcnt(0) only
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS-race debug build (compiled with -DDG_DEBUG_LDS_BARRIERS=1): after every
// phase of LDS traffic (the prologue's loads, each slab's part 1 and part 2,
// the unit's epilogue) every wave waits for all of its memory operations and
// meets a workgroup barrier.  The arithmetic is unchanged, so its results must
// equal the normal build's bit for bit; a difference means a missing wait or
// barrier in the normal schedule.  Called only where every wave arrives.
#ifndef DG_DEBUG_LDS_BARRIERS
#define DG_DEBUG_LDS_BARRIERS 0
#endif
__device__ __forceinline__ void debug_fence() {
  if constexpr (DG_DEBUG_LDS_BARRIERS != 0) {
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt, expcnt and lgkmcnt all zero
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
}

// Raw buffer descriptor: loads at byte offsets >= num_bytes return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes, 0x00020000);
}

__device__ __forceinline__ uint32_t clamp_bytes(int64_t v) {
  return v <= 0 ? 0u : (v >= 0xffffffffll ? 0xffffffffu : (uint32_t)v);
}

// BYTES (16 or 4) per lane from global (descriptor + per-lane byte offset)
// into LDS at lds_base + BYTES * lane.  The kernels wait for these loads
// with their own counted s_waitcnt.  OPAQUE issues the instruction from
// inline asm, so that the compiler does not track it: the compiler treats a
// tracked direct load as a pending write of LDS and, in kernels that also
// load into registers (the split-K reduction), makes the following LDS reads
// wait for every load in flight (s_waitcnt vmcnt(0)), which drains the
// staging pipeline.  The instruction writes no register, so nothing the
// compiler allocates can be overwritten by it late.
template <int BYTES, bool OPAQUE>
__device__ __forceinline__ void load_to_lds(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t voff) {
  static_assert(BYTES == 16 || BYTES == 4, "dwordx4 or dword");
  if constexpr (OPAQUE) {
    const uint32_t lds = (uint32_t)(uintptr_t)(lds_ptr_t)lds_base;
    if constexpr (BYTES == 16)
      asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(r), "s"(lds)
                   : "memory", "m0");
    else
      asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds" : : "v"(voff), "s"(r), "s"(lds)
                   : "memory", "m0");
  } else if constexpr (BYTES == 16) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_base, 16, voff, 0, 0, 0);
  } else {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_base, 4, voff, 0, 0, 0);
  }
}

// v_mfma_f32_16x16x128_f8f6f4, both operands E4M3 (format code 0), no block
// scaling.  out[r] for lane l = sum_k x[4*(l/16)+r][k] * y[l%16][k].
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(i32x8 x, i32x8 y) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, zero, 0, 0, 0, 0, 0, 0);
}

// Block-scaled form accumulating into c: the low byte of sx (E8M0, 2^(e-127),
// 255 = NaN) scales the 32 K-values lane l holds of x's row l%16, and sy
// likewise for y (checked on gfx950: byte 127 is 1.0, the scale of a lane
// applies to that lane's row and 32-K chunk only).
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128_e8m0(i32x8 x, i32x8 y, f32x4 c, int sx, int sy) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, c, 0, 0, 0, sx, 0, sy);
}

// Two FP32 -> BF16 conversions with v_cvt_pk_bf16_f32: round to nearest
// even, NaN stays a quiet NaN (checked bit-for-bit against the integer
// rounding u + 0x7fff + ((u >> 16) & 1) on all 2^32 inputs).
__device__ __forceinline__ uint32_t bf16x2_rne_bits(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Two 16-byte reads of a swizzled 128-byte LDS row: the lane's 32 K-bytes of
// the slab (A and B use the same K order, so the order itself is free).
__device__ __forceinline__ i32x8 read_frag(const uint8_t* row_base, int sw0, int sw1) {
  const i32x4 lo = *reinterpret_cast<const i32x4*>(row_base + sw0);
  const i32x4 hi = *reinterpret_cast<const i32x4*>(row_base + sw1);
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Renumber workgroup b so that the workgroups of one XCD (b % 8) get
// consecutive ids.
__device__ __forceinline__ int xcd_remap(int b, int grid) {
  if ((grid & 7) != 0) return b;
  return (b & 7) * (grid >> 3) + (b >> 3);
}

// Grouped raster: GM m-tiles at a time sweep the n-tiles.
template <int GM>
__device__ __forceinline__ void raster(int t, int tm, int tn, int& mb, int& nb) {
  const int per = GM * tn;
  const int grp = t / per;
  const int first = grp * GM;
  const int gsz = min(tm - first, GM);
  const int r = t - grp * per;
  mb = first + r % gsz;
  nb = r / gsz;
}

// v += C[row][gn .. gn+3] for a BF16 C (FP32 add), columns past N skipped.
// crow = element offset of the row in C.
__device__ __forceinline__ void add_c_bf16(const Params& p, int64_t crow, int gn, f32x4& v) {
  const uint16_t* C = reinterpret_cast<const uint16_t*>(p.c) + crow + gn;
  if (gn + 4 <= p.n) {  // 8-byte aligned: the row stride is a multiple of 16 bytes and gn of 4
    const uint2 cv = *reinterpret_cast<const uint2*>(C);
    v[0] += __uint_as_float(cv.x << 16);
    v[1] += __uint_as_float(cv.x & 0xFFFF0000u);
    v[2] += __uint_as_float(cv.y << 16);
    v[3] += __uint_as_float(cv.y & 0xFFFF0000u);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (gn + r < p.n) v[r] += __uint_as_float((uint32_t)C[r] << 16);
  }
}

// D[row][gn .. gn+3] = C + v (FP32 add, one rounding), columns past N dropped.
// crow / drow = element offsets of the row in C / D.
template <bool BF16_OUT, bool HAS_C>
__device__ __forceinline__ void store_out(const Params& p, int64_t crow, int gn, int64_t drow, f32x4 v) {
  const bool full = gn + 4 <= p.n;
  if (HAS_C) {
    if (BF16_OUT) {
      add_c_bf16(p, crow, gn, v);
    } else {
      const float* C = reinterpret_cast<const float*>(p.c) + crow + gn;
      if (full) {
        v += *reinterpret_cast<const f32x4*>(C);
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
      const uint32_t lo = bf16x2_rne_bits(v[0], v[1]);
      const uint32_t hi = bf16x2_rne_bits(v[2], v[3]);
      *reinterpret_cast<uint2*>(D) = make_uint2(lo, hi);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (gn + r < p.n) D[r] = (uint16_t)bf16x2_rne_bits(v[r], 0.f);
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

// E8M0: sfa/sfb hold UE8M0 bytes packed four per 32-bit word along K
// (byte j of word q = K block 4q + j): sfa words [KB/4 rounded up][ld_sfa],
// sfb words [NB][KB/4 rounded up].  Otherwise FP32 sfa [KB][ld_sfa], sfb [NB][KB].
template <int BM, int BN, int WM, int WN, int STAGES, int MODE, bool SPLIT, bool BF16_OUT, bool HAS_C, bool E8M0>
__global__ void __launch_bounds__(WM * WN * 64) gemm_kernel(const Params p) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, SFA_BYTES = BM * 4;
  // A wave's columns may straddle two 128-column scale blocks when the tile
  // width is not a multiple of 128 (or a wave's width does not divide 128).
  constexpr bool STRADDLE = (BN % 128 != 0) || (128 % TN != 0);
  // B-scale words per slab: one per 128-column block the tile can touch
  constexpr int SFB_SLOTS = STRADDLE ? (BN + 127) / 128 + 1 : (BN + 127) / 128;
  constexpr int SFB_OFF = A_BYTES + B_BYTES + SFA_BYTES;
  // stages start on 256-byte boundaries, so every stage has the same bank phase
  constexpr int STAGE = (SFB_OFF + 4 * SFB_SLOTS + 255) / 256 * 256;
  // 1 KiB (8-row) direct loads per slab: A_TOTAL of A, B_TOTAL of B, split
  // over the waves in blocks of A_LOADS / B_LOADS (the last waves may have fewer)
  constexpr int A_TOTAL = BM / 8, B_TOTAL = BN / 8;
  constexpr int A_LOADS = (A_TOTAL + NW - 1) / NW;
  constexpr int B_LOADS = (B_TOTAL + NW - 1) / NW;
  constexpr int LOADS = A_LOADS + B_LOADS;
  constexpr bool EVEN_LOADS = A_LOADS * NW == A_TOTAL && B_LOADS * NW == B_TOTAL;
  constexpr int SFA_LANES = BM / 4;  // lanes of wave 0 that stage the slab's row scales (16 B each)
  // Slab schedule (see the K loop).  The operand with fewer fragments per
  // wave ("outer": B unless A has fewer) stays in registers for the whole
  // slab; the other ("inner") is streamed.  The last HOLD inner fragments of
  // a slab are multiplied after the slab's barrier; partial t is promoted
  // after MFMA t + LAG.
  constexpr bool A_OUTER = FM < FN;
  constexpr int NO = A_OUTER ? FM : FN, NI = A_OUTER ? FN : FM;
  constexpr int HOLD = 2, FIRST = NI - HOLD;
  constexpr int T = FM * FN, T1 = FIRST * NO, P2 = HOLD * NO;
  constexpr int RING = 4, LAG = 3;
  // With two stages a slab's direct loads can start only once the previous
  // slab in its stage has been read by every wave (the barrier), and half a
  // slab's worth of loads queued at once stalls the issuing waves behind the
  // vector-memory queue.  So the loads of slab s go out in two groups: the
  // first P2L in the part 2 of slab s - 2, one per MFMA, the other P1L at the
  // first MFMAs of slab s - 1 (its stage is free then, and the barrier that
  // ends that part 1 waits for them).
  constexpr int P1L = (STAGES == 2 && LOADS / 2 <= T1) ? LOADS / 2 : 0;
  constexpr int P2L = LOADS - P1L;
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be whole 16x16 MFMA tiles");
  static_assert(TN <= 128, "a wave's columns touch at most two 128-column scale blocks");
  static_assert(FIRST >= HOLD && NO >= 2, "two-part slab schedule");
  static_assert(T % RING == 0 && LAG < RING && LAG <= P2, "promotion ring");
  static_assert(BM % 8 == 0 && BN % 8 == 0, "loads cover 8 rows");
  // uneven splits give the waves different load counts per slab, which only
  // the double-buffered schedule (it waits for all loads) tolerates
  static_assert(EVEN_LOADS || STAGES == 2, "uneven load split needs two stages");
  static_assert(SFA_LANES >= 1 && SFA_LANES <= 64 && SFA_LANES * 16 == SFA_BYTES, "sfa staging");
  static_assert(NW >= 2, "the A and B scale loads ride on different waves");
  static_assert(MODE != MODE_CONTIG || BM == 128 || BM == 256, "contiguous tiles cover one or two 128-row blocks");
  static_assert(!SPLIT || MODE == MODE_DENSE, "split-K is for dense GEMMs");
  static_assert(MODE != MODE_KGROUP || !BF16_OUT, "K-grouped outputs are FP32");
  static_assert(STAGES >= 2, "at least double buffering");

  __shared__ __attribute__((aligned(1024))) uint8_t lds[STAGES * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int KB = p.k >> 7;
  const int KQ = (KB + 3) >> 2;  // packed UE8M0 words per row
  const int NBLK = (p.n + 127) >> 7;
  const int tiles_mn = p.tiles_m * p.tiles_n;
  // lane group q reads logical K chunks q and q + 4 (measured free of LDS bank
  // conflicts on gfx950 together with the (row & 7) swizzle; chunks 2q, 2q+1 are 2-way)
  const int sw0 = (q4 ^ (r16 & 7)) << 4;
  const int sw1 = ((q4 + 4) ^ (r16 & 7)) << 4;
  // direct-load lane geometry: LDS byte 16*lane of a 1 KiB block = row lane/8,
  // physical chunk lane%8, which holds logical chunk (lane%8) ^ (lane/8).
  const int ld_row = lane >> 3;
  const int ld_chunk = ((lane & 7) ^ (lane >> 3)) << 4;

  // Work units: (tile, pass); a contiguous tile whose two 128-row halves
  // belong to different groups takes one pass per group.
  struct Unit {
    int tile, pass, passes;  // tile < 0: no unit
    int g, g0, g1, m0, n0, row_end, kb_begin, kb_end, split, tmn;  // tmn: output tile within the group
  };
  // The unit (tile, pass), or the first valid one at or after it in this
  // workgroup's tile sequence.
  // Group data (contiguous row groups, masked row counts, K sizes) is read-only
  // for the kernel, and the unit decode reads it at uniform indices: through the
  // constant address space those reads are scalar loads, which do not share the
  // vector-memory counter with the slabs in flight (as vector loads each of them
  // made the next unit's decode wait for every load issued before it).
  const __attribute__((address_space(4))) int32_t* grp_s = (const __attribute__((address_space(4))) int32_t*)p.grp;
  auto find_unit = [&](int tile, int pass) {
    Unit u;
    u.tile = -1;
    for (; tile < p.num_tiles; tile += gridDim.x, pass = 0) {
      int g = 0, t = tile, split = 0;
      if (MODE == MODE_MASKED || MODE == MODE_KGROUP) {
        g = t / tiles_mn;
        t -= g * tiles_mn;
      }
      if (SPLIT) {
        split = t / tiles_mn;
        t -= split * tiles_mn;
      }
      int kb_begin = SPLIT ? split * p.slabs_per_split : 0;
      int kb_end = SPLIT ? min(KB, kb_begin + p.slabs_per_split) : KB;
      if (MODE == MODE_KGROUP) {
        // group g's K blocks start after the blocks of groups 0..g-1; sizes are
        // device data, so they are clamped into [0, KB] rather than trusted
        int off = 0;
        for (int h = 0; h < g; ++h) off += max(grp_s[h], 0) >> 7;
        kb_begin = min(off, KB);
        kb_end = min(kb_begin + (max(grp_s[g], 0) >> 7), KB);
      }
      int mb, nb;
      raster<4>(t, p.tiles_m, p.tiles_n, mb, nb);
      const int m0 = mb * BM, n0 = nb * BN;
      // groups served by this tile (contiguous: one per 128-row half)
      int row_end = p.m, g0 = 0, g1 = 0, passes = 1;
      if (MODE == MODE_MASKED) {
        const int mm = min(max(grp_s[g], 0), p.m);
        if (m0 >= mm) continue;
        row_end = mm;
      } else if (MODE == MODE_CONTIG) {
        g0 = grp_s[m0];
        g1 = (BM == 256 && m0 + 128 < p.m) ? grp_s[m0 + 128] : -1;
        if (g0 < 0 || g0 >= p.num_groups) g0 = -1;
        if (g1 < 0 || g1 >= p.num_groups) g1 = -1;
        if (g0 < 0 && g1 < 0) continue;
        if (g0 < 0) g0 = g1;
        if (g1 < 0) g1 = g0;
        passes = (g0 == g1) ? 1 : 2;
        g = pass == 0 ? g0 : g1;
      }
      u.tile = tile;
      u.pass = pass;
      u.passes = passes;
      u.g = g;
      u.g0 = g0;
      u.g1 = g1;
      u.m0 = m0;
      u.n0 = n0;
      u.row_end = row_end;
      u.kb_begin = kb_begin;
      u.kb_end = kb_end;
      u.split = split;
      u.tmn = t;
      break;
    }
    return u;
  };
  auto next_unit = [&](const Unit& u) {
    return u.pass + 1 < u.passes ? find_unit(u.tile, u.pass + 1) : find_unit(u.tile + (int)gridDim.x, 0);
  };

  // Operand bases of a unit.
  struct Src {
    const uint8_t* A;
    const float* SFA;
    const uint8_t* B;
    const float* SFB;
    int64_t a_rows, b_rows;
    uint32_t sfb_off;
  };
  constexpr bool B_GROUPED = MODE == MODE_CONTIG || MODE == MODE_MASKED;
  const int sfb_row = E8M0 ? KQ : KB;
  const uint32_t sfb_bytes = (uint32_t)(NBLK * sfb_row) * 4;
  auto src_of = [&](const Unit& u) {
    Src r;
    r.A = p.a + (MODE == MODE_MASKED ? (int64_t)u.g * p.a_gs : 0) + (int64_t)u.m0 * p.lda;
    r.SFA = p.sfa + (MODE == MODE_MASKED ? (int64_t)u.g * p.sfa_gs : 0) + u.m0;
    r.B = p.b + (B_GROUPED ? (int64_t)u.g * p.b_gs : 0) + (int64_t)u.n0 * p.ldb;
    r.SFB = p.sfb + (B_GROUPED ? (int64_t)u.g * p.sfb_gs : 0);
    // masked groups: A rows at or past masked_m are read as zeros without touching
    // memory (their outputs are never written and no other row depends on them)
    r.a_rows = (MODE == MODE_MASKED ? u.row_end : p.m) - u.m0;
    r.b_rows = p.n - u.n0;
    // B-scale words staged with each slab: slot v holds block min(n0/128 + v, NBLK-1)
    // (clamped: columns past N are never stored)
    r.sfb_off = (uint32_t)(min((u.n0 >> 7) + lane, NBLK - 1) * sfb_row) * 4;
    return r;
  };

  // per-lane offsets of this wave's direct loads (fixed over K and tiles)
  // (loads of a wave past A_TOTAL / B_TOTAL are not issued)
  uint32_t a_off[A_LOADS], b_off[B_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) a_off[i] = (uint32_t)(((wave * A_LOADS + i) * 8 + ld_row) * p.lda) + ld_chunk;
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) b_off[i] = (uint32_t)(((wave * B_LOADS + i) * 8 + ld_row) * p.ldb) + ld_chunk;

  // Descriptors of slab kb; a slab past the unit's K range gets empty
  // descriptors, so its loads (issued anyway, which keeps the wait counts
  // fixed) fetch nothing and write zeros.
  struct SlabRsrc {
    __amdgpu_buffer_rsrc_t ra, rb;
    int kb;
    bool live;
  };
  auto slab_rsrc = [&](const Src& sr, int kb, bool live) {
    SlabRsrc r;
    r.ra = make_rsrc(sr.A + kb * 128, live ? clamp_bytes(sr.a_rows * p.lda - kb * 128) : 0u);
    r.rb = make_rsrc(sr.B + kb * 128, live ? clamp_bytes(sr.b_rows * p.ldb - kb * 128) : 0u);
    r.kb = kb;
    r.live = live;
    return r;
  };
  // Load idx of the wave's LOADS direct loads of a slab into `stage`
  // (idx < A_LOADS: A rows, else B rows); idx 0 also stages the scales
  // (A row scales on wave 0, B block scales on the last wave).
  auto issue_load = [&](const Src& sr, const SlabRsrc& r, int stage, int idx) {
    uint8_t* base = lds + stage * STAGE;
    if (idx < A_LOADS) {
      if (EVEN_LOADS || wave * A_LOADS + idx < A_TOTAL)
        load_to_lds<16, SPLIT>(r.ra, base + (wave * A_LOADS + idx) * 1024, a_off[idx]);
    } else {
      if (EVEN_LOADS || wave * B_LOADS + idx - A_LOADS < B_TOTAL)
        load_to_lds<16, SPLIT>(r.rb, base + A_BYTES + (wave * B_LOADS + idx - A_LOADS) * 1024, b_off[idx - A_LOADS]);
    }
    if (idx == 0) {
      const int q = E8M0 ? (r.kb >> 2) : r.kb;  // scale row (A) / column (B) of the slab
      if (wave == 0 && lane < SFA_LANES)
        load_to_lds<16, SPLIT>(make_rsrc(sr.SFA + (int64_t)q * p.ld_sfa, r.live ? clamp_bytes(sr.a_rows * 4) : 0u),
                               base + A_BYTES + B_BYTES, lane * 16);
      if (wave == NW - 1 && lane < SFB_SLOTS)
        load_to_lds<4, SPLIT>(make_rsrc(sr.SFB + q, r.live ? clamp_bytes((int64_t)sfb_bytes - 4 * q) : 0u),
                              base + SFB_OFF, sr.sfb_off);
    }
  };
  auto issue_slab = [&](const Src& sr, int kb, int stage, bool live) {
    const SlabRsrc r = slab_rsrc(sr, kb, live);
#pragma unroll
    for (int idx = 0; idx < LOADS; ++idx) issue_load(sr, r, stage, idx);
  };
  // Wait until this wave's loads of the slab STAGES-2 slabs before the
  // newest issued one have landed (waves 0 and NW-1 issue one more load per slab).
  auto wait_slab = [&]() {
    if (wave == 0 || wave == NW - 1) {
      wait_vmcnt<(STAGES - 2) * (LOADS + 1)>();
    } else {
      wait_vmcnt<(STAGES - 2) * LOADS>();
    }
  };

  // Cross-unit prefetch (two stages only): once a unit's K loop is done, the
  // first two slabs of the next unit are issued before the unit's epilogue,
  // so their latency hides behind the stores.  The next unit's first wait
  // then covers the stores as well (loads and stores share the vector-memory
  // counter); letting the stores stay in flight past it, with counted waits,
  // measured 1 % slower on full 256-row tiles.
  constexpr bool XPRE = STAGES == 2;
  // BF16 output: paired 16-byte stores (see the epilogue)
  constexpr bool PAIRED_STORES = BF16_OUT;
  // C enters the accumulators at the unit's start (split units: added by the reducing unit)
  constexpr bool C_FIRST = HAS_C && !SPLIT;
  constexpr bool C_LAST = HAS_C && !C_FIRST;

  const int vb = xcd_remap(blockIdx.x, gridDim.x);
  Unit u = find_unit(vb, 0), nx;
  int pre = 0;  // 0: nothing prefetched; 1: slabs 0, 1 of this unit prefetched
  while (u.tile >= 0) {
    int pre_next = 0;
    {
      const int g = u.g, m0 = u.m0, n0 = u.n0, row_end = u.row_end;
      const int kb_begin = u.kb_begin, kb_end = u.kb_end;
      const int nkb = kb_end - kb_begin;
      const int g_half[2] = {u.g0, u.g1};
      // rows this wave computes: [m0 + wm*TM, +TM); skip waves with no live rows
      const int wrow0 = m0 + wm * TM;
      bool wave_live = wrow0 < row_end;
      if (MODE == MODE_CONTIG && BM == 256) wave_live = wave_live && (g_half[(wm * TM) >> 7] == g);
      const Src sr = src_of(u);
      (void)g;

      f32x4 acc[FM][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      // C goes into the accumulators before the K loop (one batch of loads, covered
      // by the unit's first wait), not into the epilogue, where each C load would
      // wait alone behind the stores and prefetches in flight.  Split units leave C
      // to the unit that finishes the tile.
      if constexpr (C_FIRST) {
        // A tile wholly inside D (every row and column of it valid) loads C in one
        // batch with no branches; with a branch around each load (the edge tests
        // below) the compiler waited for the loads a few at a time.  Same values
        // either way: FP32 C is assigned, BF16 C added to the zeroed accumulators.
        const bool inside = m0 + BM <= row_end && n0 + BN <= p.n;
        if (wave_live && inside) {
          const int row0 = wrow0 + r16;
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const int64_t crow = (MODE == MODE_KGROUP ? (int64_t)g * p.c_gs : 0) + (int64_t)(row0 + i * 16) * p.ldc;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const int gn = n0 + wn * TN + j * 16 + 4 * q4;
              if constexpr (BF16_OUT) {
                const uint2 cv = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(p.c) + crow + gn);
                acc[i][j][0] += __uint_as_float(cv.x << 16);
                acc[i][j][1] += __uint_as_float(cv.x & 0xFFFF0000u);
                acc[i][j][2] += __uint_as_float(cv.y << 16);
                acc[i][j][3] += __uint_as_float(cv.y & 0xFFFF0000u);
              } else {
                acc[i][j] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p.c) + crow + gn);
              }
            }
          }
        } else if (wave_live) {
          int row0 = wrow0 + r16;
          asm volatile("" : "+v"(row0));
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const int gm = row0 + i * 16;
            if (gm >= row_end) continue;
            const int64_t crow = (MODE == MODE_KGROUP ? (int64_t)g * p.c_gs : 0) + (int64_t)gm * p.ldc;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const int gn = n0 + wn * TN + j * 16 + 4 * q4;
              if (gn >= p.n) continue;
              if constexpr (BF16_OUT) {
                add_c_bf16(p, crow, gn, acc[i][j]);
              } else {
                const float* C = reinterpret_cast<const float*>(p.c) + crow + gn;
                if (gn + 4 <= p.n) {
                  acc[i][j] = *reinterpret_cast<const f32x4*>(C);
                } else {
#pragma unroll
                  for (int r = 0; r < 4; ++r)
                    if (gn + r < p.n) acc[i][j][r] = C[r];
                }
              }
            }
          }
        }
        // every path into the K loop or straight to the epilogue (no slabs) sees C landed;
        // the unit's first wait covers the same loads anyway
        wait_vmcnt<0>();
      }

      // K loop.  One workgroup barrier per slab, placed inside the slab's
      // MFMAs.  The outer fragments (the operand with fewer fragments per wave)
      // stay in registers for the slab; the inner ones are streamed.  Part 1
      // multiplies inner fragments 0 .. FIRST-1 (inner-major), streaming them
      // from LDS, and reads the last HOLD inner fragments into registers; at
      // the barrier every wave has finished reading slab `it` (its stage takes
      // slab it + STAGES) and slab it + 1 has landed; part 2 multiplies the HOLD
      // held fragments (outer-major) from registers only, issuing one direct
      // load of slab it + STAGES per MFMA (with two stages only the first P2L;
      // the rest go out at the start of the next part 1) and reading slab
      // it + 1's outer fragments and first inner fragment as they free up.  No
      // LDS latency and no burst of loads sits at the barrier.  Each slab's FP32
      // promotion trails its MFMAs by LAG and carries across the slab boundary.
      // inner / outer fragment of the slab's MFMA t (part 1: inner-major over
      // the streamed fragments, part 2: outer-major over the held ones), and
      // the output fragment row / column they give
      auto inner_of = [](int t) { return t < T1 ? t / NO : FIRST + (t - T1) % HOLD; };
      auto outer_of = [](int t) { return t < T1 ? t % NO : (t - T1) / HOLD; };
      auto row_of = [&](int t) { return A_OUTER ? outer_of(t) : inner_of(t); };
      auto col_of = [&](int t) { return A_OUTER ? inner_of(t) : outer_of(t); };
      if (nkb > 0) {
        if (pre == 0) {
#pragma unroll
          for (int i = 0; i < STAGES - 1; ++i) issue_slab(sr, kb_begin + i, i, i < nkb);
          wait_slab();
        } else {
          wait_vmcnt<0>();
        }
        stage_barrier();
        if (pre == 0) issue_slab(sr, kb_begin + STAGES - 1, STAGES - 1, STAGES - 1 < nkb);
        debug_fence();

        const uint8_t* As0 = lds + (wm * TM + r16) * 128;
        const uint8_t* Bs0 = lds + A_BYTES + (wn * TN + r16) * 128;
        const uint8_t* Is0 = A_OUTER ? Bs0 : As0;  // inner operand rows
        const uint8_t* Os0 = A_OUTER ? As0 : Bs0;  // outer operand rows
        const uint8_t* Ss0 = lds + A_BYTES + B_BYTES + (wm * TM + r16) * 4;
        // this wave's first scale block (slot of the staged words) and, when
        // its columns straddle two blocks, the number of its fragments in the first
        const int wcol = n0 + wn * TN;
        const uint8_t* Sb0 = lds + SFB_OFF + ((wcol >> 7) - (n0 >> 7)) * 4;
        const int jsplit = STRADDLE ? min(FN, (128 - (wcol & 127)) >> 4) : FN;

        // slab 0's fragments, read in the order part 2 reads the next slab's,
        // so that the waits at the loop head agree on both paths into it
        i32x8 fo[NO], fh[HOLD];
        fo[0] = read_frag(Os0, sw0, sw1);
        i32x8 fi = read_frag(Is0, sw0, sw1), fi_next = fi;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int o = 1; o < NO; ++o) {
          fo[o] = read_frag(Os0 + o * 16 * 128, sw0, sw1);
          __builtin_amdgcn_sched_barrier(0);
        }
        // promotion ring; before the first slab the "previous slab's tail"
        // is 0 * 0, which leaves the zero accumulators unchanged
        f32x4 part[RING];
#pragma unroll
        for (int r = 0; r < RING; ++r) part[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        float s_tail[LAG];
#pragma unroll
        for (int l = 0; l < LAG; ++l) s_tail[l] = 0.f;

        for (int it = 0; it < nkb; ++it) {
          const int kb = kb_begin + it;
          const int cur = it % STAGES, nxt = (it + 1) % STAGES;
          const uint8_t* Is = Is0 + cur * STAGE;
          // the slab's scales (FP32: row scales and block scale; UE8M0: packed words)
          float sc[FM];
#pragma unroll
          for (int i = 0; i < FM; ++i) sc[i] = *reinterpret_cast<const float*>(Ss0 + cur * STAGE + i * 16 * 4);
          const float sb = *reinterpret_cast<const float*>(Sb0 + cur * STAGE);
          const float sb1 = STRADDLE ? *reinterpret_cast<const float*>(Sb0 + 4 + cur * STAGE) : sb;
          // s / s1: promotion scales of the wave's fragments in its first / second block
          float s[FM], s1[FM];
          int sx[FM];
          int sbx = 0, sbx1 = 0;
          if constexpr (E8M0) {
            const int sh = 8 * (kb & 3);
            sbx = (int)(__float_as_uint(sb) >> sh);
            sbx1 = (int)(__float_as_uint(sb1) >> sh);
#pragma unroll
            for (int i = 0; i < FM; ++i) sx[i] = (int)(__float_as_uint(sc[i]) >> sh);
          } else {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
              s[i] = sc[i] * sb;
              if (STRADDLE) s1[i] = sc[i] * sb1;
            }
          }
          // MFMA t of the slab with operands (outer fragment x, inner fragment y)
          auto mma = [&](int t, const i32x8& x, const i32x8& y) {
            const int i = row_of(t), j = col_of(t);
            const i32x8& fbv = A_OUTER ? y : x;  // B fragment (first operand)
            const i32x8& fav = A_OUTER ? x : y;  // A fragment
            if constexpr (E8M0) {
              acc[i][j] = mfma_fp8_16x16x128_e8m0(fbv, fav, acc[i][j], (STRADDLE && j >= jsplit) ? sbx1 : sbx, sx[i]);
            } else {
              part[t % RING] = mfma_fp8_16x16x128(fbv, fav);
            }
          };
          // acc += partial of MFMA u of this slab (u >= 0) or of the previous slab's tail (u < 0)
          auto promote = [&](int u) {
            if constexpr (!E8M0) {
              const int v = u < 0 ? u + T : u;
              const int ui = row_of(v), uj = col_of(v);
              const float su = u < 0 ? s_tail[u + LAG] : ((STRADDLE && uj >= jsplit) ? s1[ui] : s[ui]);
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[ui][uj][r] = __builtin_fmaf(part[v % RING][r], su, acc[ui][uj][r]);
            }
          };

          // the last P1L loads of slab it + 1 (slab 1 went out whole before the
          // loop, or with the previous unit's epilogue)
          const bool late_loads = P1L > 0 && it > 0;
          const SlabRsrc pr = slab_rsrc(sr, kb + 1, it + 1 < nkb);
          if (wave_live) {
#pragma unroll
            for (int t = 0; t < T1; ++t) {
              const int n = t / NO, o = t % NO;
              if (o == 0 && n + 1 < FIRST) fi_next = read_frag(Is + (n + 1) * 16 * 128, sw0, sw1);
              if (o == NO / 2 && n < HOLD) fh[n] = read_frag(Is + (FIRST + n) * 16 * 128, sw0, sw1);
              mma(t, fo[o], fi);
              promote(t - LAG);
              if (t < P1L && late_loads) issue_load(sr, pr, nxt, P2L + t);
              if (o == NO - 1 && n + 1 < FIRST) fi = fi_next;
              if (o == NO - 1) __builtin_amdgcn_sched_barrier(0);
            }
          } else if (late_loads) {
#pragma unroll
            for (int idx = P2L; idx < LOADS; ++idx) issue_load(sr, pr, nxt, idx);
          }

          debug_fence();
          // slab it + 1 has landed (this wave's part of it)
          wait_slab();
          stage_barrier();
          const bool load_live = it + STAGES < nkb;
          const SlabRsrc nr = slab_rsrc(sr, kb + STAGES, load_live);
          const uint8_t* In = Is0 + nxt * STAGE;
          const uint8_t* On = Os0 + nxt * STAGE;
          if (wave_live) {
            // (after the last slab these reads of the next stage are stale and unused)
#pragma unroll
            for (int t = T1; t < T; ++t) {
              const int w = t - T1, o = w / HOLD, h = w % HOLD;
              mma(t, fo[o], fh[h]);
              promote(t - LAG);
              if (w < P2L) issue_load(sr, nr, cur, w);
              if (h == HOLD - 1) {
                fo[o] = read_frag(On + o * 16 * 128, sw0, sw1);
                if (o == 0) fi = read_frag(In, sw0, sw1);
                __builtin_amdgcn_sched_barrier(0);
              }
            }
            if constexpr (!E8M0) {
#pragma unroll
              for (int l = 0; l < LAG; ++l) {
                const int v = T - LAG + l;
                s_tail[l] = (STRADDLE && col_of(v) >= jsplit) ? s1[row_of(v)] : s[row_of(v)];
              }
            }
          } else {
#pragma unroll
            for (int idx = 0; idx < (P2L < P2 ? P2L : P2); ++idx) issue_load(sr, nr, cur, idx);
          }
#pragma unroll
          for (int idx = P2; idx < P2L; ++idx) issue_load(sr, nr, cur, idx);
          debug_fence();
        }
        // promote the last slab's tail
        if (wave_live) {
#pragma unroll
          for (int l = 0; l < LAG; ++l) {
            if constexpr (!E8M0) {
              const int v = T - LAG + l;
              const int ui = row_of(v), uj = col_of(v);
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[ui][uj][r] = __builtin_fmaf(part[v % RING][r], s_tail[l], acc[ui][uj][r]);
            }
          }
        }
      }
      stage_barrier();  // all LDS reads of this unit are done before the next unit's loads
      debug_fence();

      // Contiguous: the group of each row this lane stores, loaded before the next
      // unit's slabs are prefetched (the vector-memory counter completes in issue
      // order, so loaded in the epilogue they waited for the prefetched slabs too).
      // Every lane loads, at a clamped row, so that no load sits in a branch (which
      // made the compiler wait for each); the epilogue's row test rejects rows past
      // row_end.
      int row_grp[MODE == MODE_CONTIG ? FM : 1];
      if constexpr (MODE == MODE_CONTIG) {
        const int row0 = wrow0 + r16;
#pragma unroll
        for (int i = 0; i < FM; ++i) row_grp[i] = p.grp[min(row0 + i * 16, row_end - 1)];
        asm volatile("" ::: "memory");  // the loads above precede the prefetch below
      }

      // next unit: its first two slabs go out before this unit's stores
      nx = next_unit(u);
      if constexpr (XPRE) {
        // Issued on every path, with empty descriptors when there is no next unit,
        // so that the loads in flight are the same wherever the compiler counts the
        // epilogue's waits (with the prefetch in a branch it fell back to waiting for
        // most of it).  The stages are free: every wave is past the last barrier.
        const bool has_next = nx.tile >= 0 && nx.kb_end > nx.kb_begin;
        const Src ns = src_of(has_next ? nx : u);
        const int kb0 = has_next ? nx.kb_begin : u.kb_begin;
        issue_slab(ns, kb0, 0, has_next);
        issue_slab(ns, kb0 + 1, 1, has_next && nx.kb_begin + 1 < nx.kb_end);
        pre_next = has_next ? 1 : 0;
        asm volatile("" ::: "memory");  // the prefetch precedes every store below
      }

      // Split K: publish this unit's partial and count it; only the unit that
      // completes its tile goes on to the epilogue, with the sum of all partials.
      bool epilogue = true;
      if constexpr (SPLIT) {
        if (p.splits > 1) {
          __shared__ int s_last;
          // Partials are stored and loaded with device-scope cache policy (sc1):
          // the stores write through to the device's point of coherence and the
          // loads read from it, so the units of one tile may run on different
          // XCDs (whose L2 caches are not coherent with each other) and no L2
          // write-back or invalidation is needed.  A unit's partial is complete
          // at that point once its stores have been acknowledged (vmcnt 0).
          constexpr int SC1 = 16;  // cache-policy bit of device-scope accesses
          constexpr int64_t TILE_ELEMS = (int64_t)BM * BN;
          const uint32_t loff = (uint32_t)(wave * FM * FN * 64 + lane) * 16;
          auto unit_rsrc = [&](int s) {
            return make_rsrc(p.ws + ((int64_t)s * tiles_mn + u.tmn) * TILE_ELEMS, (uint32_t)(TILE_ELEMS * 4));
          };
          if (wave_live) {
            const auto rw = unit_rsrc(u.split);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
              for (int j = 0; j < FN; ++j)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, acc[i][j]), rw,
                                                       loff + (i * FN + j) * 1024, 0, SC1);
          }
          wait_vmcnt<0>();
          __syncthreads();  // every wave's partial has reached the point of coherence
          if (tid == 0) {
            const uint32_t arrived =
                __hip_atomic_fetch_add(p.ctr + u.tmn, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
            const int last = arrived >= (uint32_t)p.splits;
            if (last) __hip_atomic_store(p.ctr + u.tmn, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last = last;
          }
          __syncthreads();
          epilogue = s_last != 0;
          if (epilogue && wave_live) {
            // acc = partial 0 + partial 1 + ... in split order: this unit's own
            // partial from registers, the others read back from the workspace, two
            // in flight (one CU's read rate, not the latency, bounds this loop).
            // The own partial's fetch gets an empty descriptor (no memory access), so
            // every step issues the same loads and the compiler's waits stay counted.
            constexpr int RD = 2;
            f32x4 own[FM][FN], buf[RD][FM][FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
              for (int j = 0; j < FN; ++j) own[i][j] = acc[i][j];
            auto fetch = [&](int s, f32x4 (&dst)[FM][FN]) {
              const auto rs = (s < p.splits && s != u.split) ? unit_rsrc(s) : make_rsrc(p.ws, 0u);
#pragma unroll
              for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                  dst[i][j] = __builtin_bit_cast(
                      f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, loff + (i * FN + j) * 1024, 0, SC1));
            };
#pragma unroll
            for (int r = 0; r < RD; ++r) fetch(r, buf[r]);
            for (int s0 = 0; s0 < p.splits; s0 += RD) {
#pragma unroll
              for (int r = 0; r < RD; ++r) {
                const int s = s0 + r;
                if (s < p.splits) {
                  const bool mine = s == u.split;
#pragma unroll
                  for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                      const f32x4 v = mine ? own[i][j] : buf[r][i][j];
                      acc[i][j] = s == 0 ? v : acc[i][j] + v;
                    }
                }
                fetch(s + RD, buf[r]);
              }
            }
          }
          wait_vmcnt<0>();
        }
      }

      if (wave_live && epilogue) {
        // Epilogue: D = C + acc, masked stores.  (The empty asm makes the row
        // index opaque, so the row addresses are computed here instead of being
        // hoisted above the K loop, where registers are scarce.)
        int row0 = wrow0 + r16;
        asm volatile("" : "+v"(row0));
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int gm = row0 + i * 16;
          bool row_ok = gm < row_end;
          if constexpr (MODE == MODE_CONTIG) row_ok = row_ok && row_grp[i] == g;
          const int64_t drow = (MODE == MODE_MASKED || MODE == MODE_KGROUP ? (int64_t)g * p.d_gs : 0) + (int64_t)gm * p.ldd;
          const int64_t crow = (MODE == MODE_KGROUP ? (int64_t)g * p.c_gs : 0) + (int64_t)gm * p.ldc;
          if constexpr (PAIRED_STORES) {
            // Adjacent column fragments j, j+1 in BF16: one permlane16 swap per
            // word pair leaves each lane 8 consecutive columns of its row
            // (16-lane row q4 even: fragment j, odd: j+1; columns 8 * (q4 / 2) ..),
            // so a row's 64 bytes go out as four 16-byte stores instead of eight
            // of 8 bytes.  The swap partners share r16, hence the row and its
            // row_ok; the swaps run before the row test, on the whole wave.
#pragma unroll
            for (int j = 0; j + 1 < FN; j += 2) {
              if (C_LAST && row_ok) {  // C in the MFMA layout: this lane's row, columns 4 * q4 ..
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                  const int gc = n0 + wn * TN + (j + h) * 16 + 4 * q4;
                  if (gc < p.n) add_c_bf16(p, crow, gc, acc[i][j + h]);
                }
              }
              const auto s0 = __builtin_amdgcn_permlane16_swap(bf16x2_rne_bits(acc[i][j][0], acc[i][j][1]),
                                                               bf16x2_rne_bits(acc[i][j + 1][0], acc[i][j + 1][1]),
                                                               false, false);
              const auto s1 = __builtin_amdgcn_permlane16_swap(bf16x2_rne_bits(acc[i][j][2], acc[i][j][3]),
                                                               bf16x2_rne_bits(acc[i][j + 1][2], acc[i][j + 1][3]),
                                                               false, false);
              const int gn = n0 + wn * TN + (j + (q4 & 1)) * 16 + 8 * (q4 >> 1);
              if (!row_ok || gn >= p.n) continue;
              uint16_t* D = reinterpret_cast<uint16_t*>(p.d) + drow + gn;
              const uint32_t w[4] = {s0[0], s1[0], s0[1], s1[1]};
              if (gn + 8 <= p.n) {
                *reinterpret_cast<uint4*>(D) = make_uint4(w[0], w[1], w[2], w[3]);
              } else {
#pragma unroll
                for (int c = 0; c < 8; ++c)
                  if (gn + c < p.n) D[c] = (uint16_t)(w[c >> 1] >> (16 * (c & 1)));
              }
            }
            if constexpr (FN % 2 == 1) {
              const int gn = n0 + wn * TN + (FN - 1) * 16 + 4 * q4;
              if (row_ok && gn < p.n) store_out<BF16_OUT, C_LAST>(p, crow, gn, drow, acc[i][FN - 1]);
            }
          } else {
            if (!row_ok) continue;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const int gn = n0 + wn * TN + j * 16 + 4 * q4;
              if (gn >= p.n) continue;
              store_out<BF16_OUT, C_LAST>(p, crow, gn, drow, acc[i][j]);
            }
          }
        }
      }
      asm volatile("" ::: "memory");  // every store precedes the next unit's first wait
      debug_fence();
    }
    u = nx;
    pre = pre_next;
  }
  wait_vmcnt<0>();  // no direct load into this workgroup's LDS outlives it
}

}  // namespace dg
