// dg_api.hip -- host side of libdg: argument validation, tile-config choice
// and kernel launch for the C ABI declared in include/dg.h.
//
// Source for the operations and their conventions: DeepGEMM README as
// mirrored on "Weight gradient kernels for dense and MoE models #95",
// sections "Interfaces > Notices", "Grouped GEMMs (contiguous layout)",
// "Grouped GEMMs (masked layout)" and "Utilities" (SM cap, contiguous-layout
// alignment, aligned scale size); the DG_PRINT_CONFIGS switch mirrors the
// README's environment variable of the same name ("General").
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "dg.h"
#include "dg_common.hpp"
#include "dg_internal.h"
#include "dg_kernels.hpp"

namespace {

constexpr int kAlignM = 128;
constexpr int kMaxDevices = 64;
// Split-K workspace layout: kCtrWords tile counters (zero between calls), then
// the FP32 partial tiles.  The counters sit at a fixed place so that calls of
// different shapes sharing one workspace never read partials as counters.
constexpr int kCtrWords = 16384;
constexpr size_t kCtrBytes = kCtrWords * sizeof(uint32_t);
constexpr size_t kWorkspaceAlign = 256;

std::atomic<int> g_num_cus{-1};  // -1: not yet read from the environment
int g_device_cus[kMaxDevices] = {0};
std::once_flag g_env_once;
bool g_print_configs = false;
std::atomic<int> g_tile_n{0};  // forced width of the 256-row tiles (0 = automatic; tests only)

void read_env() {
  std::call_once(g_env_once, [] {
    const char* s = std::getenv("DG_PRINT_CONFIGS");
    g_print_configs = s && std::atoi(s) != 0;
    int expected = -1;
    const char* c = std::getenv("DG_NUM_CUS");
    const int v = c ? std::atoi(c) : 0;
    g_num_cus.compare_exchange_strong(expected, v > 0 ? v : 0);
  });
}

dg_status hip_fail(hipError_t e) { return dg::record_hip_error(e); }

// CUs the kernels may spread over on the current device.
dg_status usable_cus(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  int total = (dev >= 0 && dev < kMaxDevices) ? g_device_cus[dev] : 0;
  if (total <= 0) {
    e = hipDeviceGetAttribute(&total, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev >= 0 && dev < kMaxDevices) g_device_cus[dev] = total;
  }
  read_env();
  const int cap = g_num_cus.load();
  *out = (cap > 0 && cap < total) ? cap : total;
  return DG_SUCCESS;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline int cdiv(int a, int b) { return (a + b - 1) / b; }
inline int64_t dtype_size(dg_dtype t) { return t == DG_DTYPE_BF16 ? 2 : 4; }

using KernelFn = void (*)(dg::Params);

// Tile configurations.  LDS per workgroup = stages x ((BM + BN) x 128 B + BM x 4 B
// + B-scale words, rounded up to 256 B):
//   256x256, 8 waves, 2 stages: 130 KiB (one workgroup per CU) -- large M and N
//   256x224, 8 waves, 2 stages: 122 KiB (one per CU)            -- large M, N = 7 x 1024
//   256x160, 8 waves, 2 stages: 106 KiB (one per CU)            -- large M, N like 2112
//   128x128, 4 waves, 2 stages:  65 KiB (two per CU)           -- small grouped tiles
//   128x64,  4 waves, 3 stages:  74 KiB (two per CU), split-K  -- dense 64 < M <= 128
//    64x128, 4 waves, 3 stages:  73 KiB (two per CU), split-K  -- dense M <= 64
// The split-K configurations stream B from HBM; two independent workgroups
// per CU keep four slabs in flight per CU.
enum TileId { TILE_256x256 = 0, TILE_128x128 = 1, TILE_SK_128x64 = 2, TILE_SK_64x128 = 3, TILE_256x224 = 4,
              TILE_256x160 = 5, TILE_SK_128x128 = 6 };

struct Cfg {
  TileId id;
  int bm, bn, wm, wn, stages, per_cu;
};

constexpr Cfg kCfg256{TILE_256x256, 256, 256, 2, 4, 2, 1};
constexpr Cfg kCfg256x224{TILE_256x224, 256, 224, 4, 2, 2, 1};
constexpr Cfg kCfg256x160{TILE_256x160, 256, 160, 4, 2, 2, 1};
constexpr Cfg kCfg128{TILE_128x128, 128, 128, 2, 2, 2, 2};
constexpr Cfg kCfgSk128{TILE_SK_128x64, 128, 64, 2, 2, 3, 2};
constexpr Cfg kCfgSk64{TILE_SK_64x128, 64, 128, 1, 4, 3, 2};
constexpr Cfg kCfgSk128x128{TILE_SK_128x128, 128, 128, 2, 2, 3, 1};

// Output flavour of a launch.
struct Epi {
  bool bf16, has_c, e8m0;
};

// Only the combinations the entry points can reach are instantiated:
// dense: every tile, BF16/FP32, with/without C (the skinny tiles split K);
// M-grouped: the 256-row tiles and 128x128 without C; K-grouped: FP32
// with/without C.
template <int BM, int BN, int WM, int WN, int ST, int MODE, bool E8M0, bool SPLIT_TILE = false>
KernelFn pick_out(const Epi& e) {
  constexpr bool kSplit = MODE == dg::MODE_DENSE && (SPLIT_TILE || BM < 128 || BN < 128);
  if constexpr (MODE == dg::MODE_DENSE) {
    if (e.bf16)
      return e.has_c ? dg::gemm_kernel<BM, BN, WM, WN, ST, MODE, kSplit, true, true, E8M0>
                     : dg::gemm_kernel<BM, BN, WM, WN, ST, MODE, kSplit, true, false, E8M0>;
    return e.has_c ? dg::gemm_kernel<BM, BN, WM, WN, ST, MODE, kSplit, false, true, E8M0>
                   : dg::gemm_kernel<BM, BN, WM, WN, ST, MODE, kSplit, false, false, E8M0>;
  } else if constexpr (MODE == dg::MODE_KGROUP) {
    return e.has_c ? dg::gemm_kernel<BM, BN, WM, WN, ST, MODE, false, false, true, E8M0>
                   : dg::gemm_kernel<BM, BN, WM, WN, ST, MODE, false, false, false, E8M0>;
  } else {
    return e.bf16 ? dg::gemm_kernel<BM, BN, WM, WN, ST, MODE, false, true, false, E8M0>
                  : dg::gemm_kernel<BM, BN, WM, WN, ST, MODE, false, false, false, E8M0>;
  }
}

template <int MODE, bool E8M0>
KernelFn pick_tile(const Cfg& c, const Epi& e) {
  if constexpr (MODE == dg::MODE_DENSE) {
    if (c.id == TILE_SK_128x64) return pick_out<128, 64, 2, 2, 3, MODE, E8M0>(e);
    if (c.id == TILE_SK_64x128) return pick_out<64, 128, 1, 4, 3, MODE, E8M0>(e);
    if (c.id == TILE_SK_128x128) return pick_out<128, 128, 2, 2, 3, MODE, E8M0, true>(e);
  }
  if (c.id == TILE_256x256) return pick_out<256, 256, 2, 4, 2, MODE, E8M0>(e);
  if (c.id == TILE_256x224) return pick_out<256, 224, 4, 2, 2, MODE, E8M0>(e);
  if (c.id == TILE_256x160) return pick_out<256, 160, 4, 2, 2, MODE, E8M0>(e);
  return pick_out<128, 128, 2, 2, 2, MODE, E8M0>(e);
}

template <int MODE>
KernelFn pick_kernel(const Cfg& c, const Epi& e) {
  return e.e8m0 ? pick_tile<MODE, true>(c, e) : pick_tile<MODE, false>(c, e);
}

const char* mode_name(int mode) {
  return mode == dg::MODE_DENSE ? "dense" : mode == dg::MODE_CONTIG ? "contiguous"
       : mode == dg::MODE_MASKED ? "masked" : "k-grouped";
}

// Width of the 256-row tiles: the candidate with the least (workgroup rounds x
// tile width x relative cost per column) -- narrower tiles even out the last
// round of tiles (N = 7168: 448 tiles of 256x256 on 256 CUs leave 1.75 rounds,
// 512 tiles of 256x224 exactly 2) but re-read more LDS per MFMA.
// `row_tiles` = 256-row tiles per N column of tiles (all groups together).
Cfg choose_wide(int64_t row_tiles, int n, int slots) {
  read_env();
  const Cfg cands[3] = {kCfg256, kCfg256x224, kCfg256x160};
  // time per tile column relative to 256x256 (time per round of tiles divided
  // by the tile width: 1.02 and 1.09 on 8192x8192x16384; the 256x224 tile
  // measured ~1.04 on the contiguous MoE workload)
  const double col_cost[3] = {1.0, 1.04, 1.09};
  Cfg best = kCfg256;
  double best_cost = 1e300;
  for (int i = 0; i < 3; ++i) {
    const int forced = g_tile_n.load();
    if (forced > 0 && cands[i].bn != forced) continue;
    const int64_t tiles = row_tiles * cdiv(n, cands[i].bn);
    const int64_t rounds = (tiles + slots - 1) / slots;
    const double cost = static_cast<double>(rounds) * cands[i].bn * col_cost[i];
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = cands[i];
    }
  }
  return best;
}

// Skinny dense GEMMs (M <= 128) split K over workgroups.  Estimated time of a
// (tile, splits) candidate, in microseconds, from per-unit timelines taken with
// s_memrealtime stamps on MI355X: ~2.5 us from launch to a unit's first slab,
// then one slab per (BM + BN) x 128 B / 36 GB/s (what one CU sustains for these
// row-strided direct loads, whatever the ring depth), ~1.7 us to publish a
// partial, and the last unit of a tile reading every partial at ~85 GB/s.
// Units beyond one per CU wait for a round (two on one CU share its loads).
// A 128-column tile reads each A slab half as often per B byte as a 64-column
// one but makes fewer tiles (more splits) and larger partials.
double skinny_cost(const Cfg& c, int64_t tiles, int kb, int s, int cus) {
  const int sps = cdiv(kb, s);
  const int64_t rounds = (tiles * s + cus - 1) / cus;
  const double slab_us = (c.bm + c.bn) * 128.0 / 36e3;
  double unit_us = 2.5 + (sps - 1) * slab_us;
  double tail_us = 0.0;
  if (s > 1) {
    unit_us += 1.7;
    tail_us = s * static_cast<double>(c.bm) * c.bn * sizeof(float) / 85e3;
  }
  return static_cast<double>(rounds) * unit_us + tail_us;
}

// Partials of one call: at most 16 MiB (two 128x64 / 64x128 units or one
// 128x128 unit per CU of a 256-CU device), which is also the allocation-free
// entry point's scratch, so both entry points make the same plans.
constexpr size_t kMaxPartialBytes = size_t(16) << 20;

// Tile configuration and K split of a dense call, and the workspace the split needs.
struct DensePlan {
  Cfg cfg;
  int splits, slabs_per_split;
  size_t ws_bytes;  // 0: no split, no workspace
};

// The plan on a device with `cus` usable CUs (host arithmetic only).
DensePlan plan_dense_for(int m, int n, int k, int cus) {
  DensePlan pl{};
  pl.splits = 1;
  pl.slabs_per_split = k / 128;
  pl.ws_bytes = 0;
  if (m > 128) {
    pl.cfg = n > 128 ? choose_wide(cdiv(m, 256), n, cus) : kCfg128;
    return pl;
  }
  // Skinny: every candidate tile and split count (splits that would put more than
  // two units on a CU are not considered: splitting pays only while tiles leave CUs idle).
  const Cfg cands[2] = {m <= 64 ? kCfgSk64 : kCfgSk128, kCfgSk128x128};
  const int ncand = m <= 64 ? 1 : 2;
  const int kb = k / 128;
  double best = 1e300;
  pl.cfg = cands[0];
  for (int ci = 0; ci < ncand; ++ci) {
    const Cfg& c = cands[ci];
    const int64_t tiles = static_cast<int64_t>(cdiv(m, c.bm)) * cdiv(n, c.bn);
    if (tiles <= 0) continue;
    for (int s = 1; s <= kb; ++s) {
      const int sps = cdiv(kb, s);
      if (cdiv(kb, sps) != s) continue;  // each split count once, as its slabs per split
      const size_t part = static_cast<size_t>(s) * tiles * c.bm * c.bn * sizeof(float);
      if (s > 1 && (tiles * s > 2ll * cus || part > kMaxPartialBytes || tiles > kCtrWords)) break;
      const double cost = skinny_cost(c, tiles, kb, s, cus);
      if (cost < best - 1e-9) {
        best = cost;
        pl.cfg = c;
        pl.splits = s;
        pl.slabs_per_split = sps;
        pl.ws_bytes = s > 1 ? kCtrBytes + part : 0;
      }
    }
  }
  return pl;
}

dg_status plan_dense(int m, int n, int k, DensePlan* out) {
  int cus = 0;
  dg_status st = usable_cus(&cus);
  if (st != DG_SUCCESS) return st;
  *out = plan_dense_for(m, n, k, cus);
  return DG_SUCCESS;
}

// Fills the tile grid of p and launches.  p.splits / p.slabs_per_split / p.ws /
// p.ctr are set by the caller (dense split-K) or left at one split.
template <int MODE>
dg_status launch(dg::Params& p, const Cfg& cfg, dg_dtype t, bool has_c, bool e8m0, int groups_for_tiles,
                 hipStream_t stream) {
  p.tiles_m = cdiv(p.m, cfg.bm);
  p.tiles_n = cdiv(p.n, cfg.bn);
  if (p.splits < 1) {
    p.splits = 1;
    p.slabs_per_split = p.k / 128;
  }
  int cus = 0;
  dg_status st = usable_cus(&cus);
  if (st != DG_SUCCESS) return st;
  const int slots = cus * cfg.per_cu;
  p.num_tiles = p.tiles_m * p.tiles_n * groups_for_tiles * p.splits;
  if (p.num_tiles <= 0) return DG_SUCCESS;
  const int grid = p.num_tiles < slots ? p.num_tiles : slots;
  KernelFn fn = pick_kernel<MODE>(cfg, Epi{t == DG_DTYPE_BF16, has_c, e8m0});
  if (g_print_configs)
    std::fprintf(stderr,
                 "dg: %s%s m=%d n=%d k=%d groups=%d -> BM=%d BN=%d waves=%dx%d stages=%d splits=%d (x%d slabs) "
                 "tiles=%d grid=%d cus=%d\n",
                 mode_name(MODE), e8m0 ? " ue8m0" : "", p.m, p.n, p.k, p.num_groups, cfg.bm, cfg.bn, cfg.wm, cfg.wn,
                 cfg.stages, p.splits, p.slabs_per_split, p.num_tiles, grid, cus);
  hipLaunchKernelGGL(fn, dim3(grid), dim3(cfg.wm * cfg.wn * 64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return DG_SUCCESS;
}

// Shared operand checks; rows = rows of A (M, M_total or M_max).  Both scale
// forms use 4-byte elements (FP32 values or packed UE8M0 words).
dg_status check_common(const void* a, const void* sfa, int64_t ld_sfa, const void* b, const void* sfb,
                       const void* d, dg_dtype t, int rows, int n, int k) {
  if (rows < 0 || n < 0 || k < 0) return DG_ERROR_INVALID_VALUE;
  if (t != DG_DTYPE_BF16 && t != DG_DTYPE_FP32) return DG_ERROR_INVALID_VALUE;
  if (k % 128 != 0) return DG_ERROR_NOT_SUPPORTED;
  if (d == nullptr || !aligned(d, 16)) return DG_ERROR_INVALID_VALUE;
  if (k > 0) {
    if (a == nullptr || b == nullptr || sfa == nullptr || sfb == nullptr) return DG_ERROR_INVALID_VALUE;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(sfa, 16) || !aligned(sfb, 4))
      return DG_ERROR_INVALID_VALUE;
    if (ld_sfa < rows || ld_sfa % 4 != 0) return DG_ERROR_INVALID_VALUE;
  }
  return DG_SUCCESS;
}

// Rows of sfb per 128-column block: K blocks (FP32) or packed words (UE8M0).
inline int64_t sfb_row(int k, bool e8m0) { return e8m0 ? (k / 128 + 3) / 4 : k / 128; }
// Rows of sfa per group: K blocks (FP32) or packed words (UE8M0).
inline int64_t sfa_rows(int k, bool e8m0) { return sfb_row(k, e8m0); }

dg_status dense_impl(const void* a, int64_t lda, const void* sfa, int64_t ld_sfa, const void* b, int64_t ldb,
                     const void* sfb, const void* c, int64_t ldc, void* d, int64_t ldd, dg_dtype d_dtype, int m,
                     int n, int k, bool e8m0, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  dg_status st = check_common(a, sfa, ld_sfa, b, sfb, d, d_dtype, m, n, k);
  if (st != DG_SUCCESS) return st;
  const int64_t es = dtype_size(d_dtype);
  if (k > 0 && (lda < k || ldb < k || lda % 16 != 0 || ldb % 16 != 0)) return DG_ERROR_INVALID_VALUE;
  if (ldd < n || (ldd * es) % 16 != 0) return DG_ERROR_INVALID_VALUE;
  if (c != nullptr && (!aligned(c, 16) || ldc < n || (ldc * es) % 16 != 0)) return DG_ERROR_INVALID_VALUE;
  if (m == 0 || n == 0) return DG_SUCCESS;
  if (static_cast<int64_t>(lda) * 256 >= (1ll << 31) || static_cast<int64_t>(ldb) * 256 >= (1ll << 31))
    return DG_ERROR_NOT_SUPPORTED;
  DensePlan pl{};
  st = plan_dense(m, n, k, &pl);
  if (st != DG_SUCCESS) return st;
  if (pl.ws_bytes > 0 &&
      (workspace == nullptr || !aligned(workspace, kWorkspaceAlign) || workspace_bytes < pl.ws_bytes))
    return DG_ERROR_WORKSPACE;

  dg::Params p{};
  p.a = static_cast<const uint8_t*>(a);
  p.sfa = static_cast<const float*>(sfa);
  p.b = static_cast<const uint8_t*>(b);
  p.sfb = static_cast<const float*>(sfb);
  p.c = c;
  p.d = d;
  p.grp = nullptr;
  p.lda = lda;
  p.ldb = ldb;
  p.ldc = ldc;
  p.ldd = ldd;
  p.ld_sfa = ld_sfa;
  p.m = m;
  p.n = n;
  p.k = k;
  p.num_groups = 1;
  p.splits = pl.splits;
  p.slabs_per_split = pl.slabs_per_split;
  if (pl.ws_bytes > 0) {
    p.ctr = static_cast<uint32_t*>(workspace);
    p.ws = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kCtrBytes);
  }
  return launch<dg::MODE_DENSE>(p, pl.cfg, d_dtype, c != nullptr, e8m0, 1, stream);
}

dg_status contiguous_impl(const void* a, const void* sfa, int64_t ld_sfa, const void* b, const void* sfb, void* d,
                          dg_dtype d_dtype, const int32_t* m_indices, int m_total, int n, int k, int num_groups,
                          bool e8m0, hipStream_t stream) {
  if (num_groups < 0) return DG_ERROR_INVALID_VALUE;
  dg_status st = check_common(a, sfa, ld_sfa, b, sfb, d, d_dtype, m_total, n, k);
  if (st != DG_SUCCESS) return st;
  if (m_total % kAlignM != 0) return DG_ERROR_NOT_SUPPORTED;
  if ((static_cast<int64_t>(n) * dtype_size(d_dtype)) % 16 != 0) return DG_ERROR_INVALID_VALUE;
  if (m_total == 0 || n == 0 || num_groups == 0) return DG_SUCCESS;
  if (m_indices == nullptr || !aligned(m_indices, 4)) return DG_ERROR_INVALID_VALUE;

  dg::Params p{};
  p.a = static_cast<const uint8_t*>(a);
  p.sfa = static_cast<const float*>(sfa);
  p.b = static_cast<const uint8_t*>(b);
  p.sfb = static_cast<const float*>(sfb);
  p.c = nullptr;
  p.d = d;
  p.grp = m_indices;
  p.lda = k;
  p.ldb = k;
  p.ldd = n;
  p.ld_sfa = ld_sfa;
  p.b_gs = static_cast<int64_t>(n) * k;
  p.sfb_gs = static_cast<int64_t>(cdiv(n, 128)) * sfb_row(k, e8m0);
  p.m = m_total;
  p.n = n;
  p.k = k;
  p.num_groups = num_groups;
  if (static_cast<int64_t>(k) * 256 >= (1ll << 31)) return DG_ERROR_NOT_SUPPORTED;
  int cus = 0;
  st = usable_cus(&cus);
  if (st != DG_SUCCESS) return st;
  const Cfg cfg = n > 128 ? choose_wide(cdiv(m_total, 256), n, cus) : kCfg128;
  // Ragged last round: the token count sets the number of 256-row tiles, so
  // the last round of a persistent launch can keep only a few CUs busy for a
  // whole tile time.  When it would be at most half full, the rows of that
  // round go to a second launch of 128x128 tiles (four per 256-row tile, two
  // workgroups per CU) that fits in one round.  Rows are split at a multiple
  // of 256, so every 128-row block keeps its group; the per-element sums are
  // the same, so the bits do not change.
  const int64_t col_tiles = cdiv(n, cfg.bn);
  const int64_t slots = static_cast<int64_t>(cus) * cfg.per_cu;
  const int64_t tiles = static_cast<int64_t>(cdiv(m_total, 256)) * col_tiles;
  const int64_t rounds = tiles / slots, rem = tiles % slots;
  if (cfg.bm == 256 && rounds >= 1 && rem > 0 && 2 * rem <= slots) {
    const int main_rows = static_cast<int>(rounds * slots / col_tiles) * 256;
    const int tail_rows = m_total - main_rows;
    const int64_t tail_tiles = static_cast<int64_t>(cdiv(tail_rows, 128)) * cdiv(n, 128);
    if (main_rows > 0 && tail_rows > 0 && tail_tiles <= static_cast<int64_t>(cus) * kCfg128.per_cu) {
      dg::Params q = p;
      p.m = main_rows;
      st = launch<dg::MODE_CONTIG>(p, cfg, d_dtype, false, e8m0, 1, stream);
      if (st != DG_SUCCESS) return st;
      q.a += static_cast<int64_t>(main_rows) * k;
      q.sfa += main_rows;
      q.d = static_cast<uint8_t*>(d) + static_cast<int64_t>(main_rows) * n * dtype_size(d_dtype);
      q.grp += main_rows;
      q.m = tail_rows;
      return launch<dg::MODE_CONTIG>(q, kCfg128, d_dtype, false, e8m0, 1, stream);
    }
  }
  return launch<dg::MODE_CONTIG>(p, cfg, d_dtype, false, e8m0, 1, stream);
}

dg_status masked_impl(const void* a, const void* sfa, int64_t ld_sfa, const void* b, const void* sfb, void* d,
                      dg_dtype d_dtype, const int32_t* masked_m, int num_groups, int m_max, int n, int k,
                      int expected_m, bool e8m0, hipStream_t stream) {
  if (num_groups < 0) return DG_ERROR_INVALID_VALUE;
  dg_status st = check_common(a, sfa, ld_sfa, b, sfb, d, d_dtype, m_max, n, k);
  if (st != DG_SUCCESS) return st;
  if ((static_cast<int64_t>(n) * dtype_size(d_dtype)) % 16 != 0) return DG_ERROR_INVALID_VALUE;
  if (m_max == 0 || n == 0 || num_groups == 0) return DG_SUCCESS;
  if (masked_m == nullptr || !aligned(masked_m, 4)) return DG_ERROR_INVALID_VALUE;

  dg::Params p{};
  p.a = static_cast<const uint8_t*>(a);
  p.sfa = static_cast<const float*>(sfa);
  p.b = static_cast<const uint8_t*>(b);
  p.sfb = static_cast<const float*>(sfb);
  p.c = nullptr;
  p.d = d;
  p.grp = masked_m;
  p.lda = k;
  p.ldb = k;
  p.ldd = n;
  p.ld_sfa = ld_sfa;
  p.a_gs = static_cast<int64_t>(m_max) * k;
  p.sfa_gs = sfa_rows(k, e8m0) * ld_sfa;
  p.b_gs = static_cast<int64_t>(n) * k;
  p.sfb_gs = static_cast<int64_t>(cdiv(n, 128)) * sfb_row(k, e8m0);
  p.d_gs = static_cast<int64_t>(m_max) * n;
  p.m = m_max;
  p.n = n;
  p.k = k;
  p.num_groups = num_groups;
  if (static_cast<int64_t>(k) * 256 >= (1ll << 31)) return DG_ERROR_NOT_SUPPORTED;
  const int em = expected_m > 0 ? expected_m : m_max;
  int cus = 0;
  st = usable_cus(&cus);
  if (st != DG_SUCCESS) return st;
  // Decode-sized groups stream B: one 256-row workgroup per CU keeps more of B in flight
  // than two 128x128 ones, and was faster at every expected_m measured (masked_m uniform in
  // [0, 16] up to [0, 256]; -20 to -30 % time), so 128x128 only serves n <= 128.
  const Cfg cfg = n > 128 ? choose_wide(static_cast<int64_t>(num_groups) * cdiv(em, 256), n, cus) : kCfg128;
  return launch<dg::MODE_MASKED>(p, cfg, d_dtype, false, e8m0, num_groups, stream);
}

dg_status k_grouped_impl(const void* a, const void* sfa, int64_t ld_sfa, const void* b, const void* sfb,
                         const float* c, float* d, const int32_t* ks, int num_groups, int m, int n, int k_total,
                         bool e8m0, hipStream_t stream) {
  if (num_groups < 0) return DG_ERROR_INVALID_VALUE;
  dg_status st = check_common(a, sfa, ld_sfa, b, sfb, d, DG_DTYPE_FP32, m, n, k_total);
  if (st != DG_SUCCESS) return st;
  if ((static_cast<int64_t>(n) * 4) % 16 != 0) return DG_ERROR_INVALID_VALUE;
  if (c != nullptr && !aligned(c, 16)) return DG_ERROR_INVALID_VALUE;
  if (m == 0 || n == 0 || num_groups == 0) return DG_SUCCESS;
  if (ks == nullptr || !aligned(ks, 4)) return DG_ERROR_INVALID_VALUE;

  dg::Params p{};
  p.a = static_cast<const uint8_t*>(a);
  p.sfa = static_cast<const float*>(sfa);
  p.b = static_cast<const uint8_t*>(b);
  p.sfb = static_cast<const float*>(sfb);
  p.c = c;
  p.d = d;
  p.grp = ks;
  p.lda = k_total;
  p.ldb = k_total;
  p.ldc = n;
  p.ldd = n;
  p.ld_sfa = ld_sfa;
  p.c_gs = static_cast<int64_t>(m) * n;
  p.d_gs = static_cast<int64_t>(m) * n;
  p.m = m;
  p.n = n;
  p.k = k_total;
  p.num_groups = num_groups;
  if (static_cast<int64_t>(k_total) * 256 >= (1ll << 31)) return DG_ERROR_NOT_SUPPORTED;
  int cus = 0;
  st = usable_cus(&cus);
  if (st != DG_SUCCESS) return st;
  const Cfg cfg = (m > 128 && n > 128) ? choose_wide(static_cast<int64_t>(num_groups) * cdiv(m, 256), n, cus) : kCfg128;
  return launch<dg::MODE_KGROUP>(p, cfg, DG_DTYPE_FP32, c != nullptr, e8m0, num_groups, stream);
}

// ---- allocation-free dense entry point ---------------------------------------
// Split-K scratch of dg_fp8_gemm_nt_noalloc: counters then partials, the
// largest workspace plan_dense asks for (kMaxPartialBytes of partials).  Each device holds its own copy; its address comes
// from hipGetSymbolAddress on that device (the name itself is only a host-side
// stand-in) and is kept per device.
constexpr size_t kScratchBytes = kCtrBytes + kMaxPartialBytes;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

dg_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return DG_ERROR_NOT_SUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DG_SUCCESS;
}

// Zero n counter words (a kernel, not hipMemsetAsync, so the call stays
// capturable into a graph that is replayed many times).
__global__ void __launch_bounds__(256) clear_words_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

}  // namespace

namespace dg {

thread_local char g_last_hip_error[256] = "";

dg_status record_hip_error(hipError_t e) {
  std::snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s", hipGetErrorString(e));
  return DG_ERROR_LAUNCH_FAILED;
}

}  // namespace dg

extern "C" {

dg_status dg_fp8_gemm_nt(const void* a, int64_t lda, const float* sfa, int64_t ld_sfa, const void* b,
                         int64_t ldb, const float* sfb, const void* c, int64_t ldc, void* d, int64_t ldd,
                         dg_dtype d_dtype, int m, int n, int k, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  return dense_impl(a, lda, sfa, ld_sfa, b, ldb, sfb, c, ldc, d, ldd, d_dtype, m, n, k, false, workspace,
                    workspace_bytes, stream);
}

dg_status dg_fp8_gemm_nt_noalloc(const void* a, int64_t lda, const float* sfa, int64_t ld_sfa, const void* b,
                                 int64_t ldb, const float* sfb, const void* c, int64_t ldc, void* d, int64_t ldd,
                                 dg_dtype d_dtype, int m, int n, int k, hipStream_t stream) {
  dg_status st = check_common(a, sfa, ld_sfa, b, sfb, d, d_dtype, m, n, k);
  if (st != DG_SUCCESS || m == 0 || n == 0) return st;
  DensePlan pl{};
  if (k % 128 == 0 && m > 0 && n > 0 && k > 0) {
    st = plan_dense(m, n, k, &pl);
    if (st != DG_SUCCESS) return st;
  }
  if (pl.ws_bytes > kScratchBytes) return DG_ERROR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (pl.ws_bytes > 0) {
    st = scratch_address(&ws);
    if (st != DG_SUCCESS) return st;
    // the counters of this call's tiles start at zero whatever the last call left
    const int words = cdiv(m, pl.cfg.bm) * cdiv(n, pl.cfg.bn);  // one counter per output tile
    const int grid = cdiv(words, 256) < 64 ? cdiv(words, 256) : 64;
    hipLaunchKernelGGL(clear_words_kernel, dim3(grid), dim3(256), 0, stream, static_cast<uint32_t*>(ws), words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
  }
  return dense_impl(a, lda, sfa, ld_sfa, b, ldb, sfb, c, ldc, d, ldd, d_dtype, m, n, k, false, ws,
                    ws != nullptr ? kScratchBytes : 0, stream);
}

size_t dg_get_workspace_size(int m, int n, int k) {
  if (m <= 0 || n <= 0 || k <= 0 || k % 128 != 0) return 0;
  DensePlan pl{};
  if (plan_dense(m, n, k, &pl) != DG_SUCCESS) return 0;
  return pl.ws_bytes;
}

dg_status dg_m_grouped_fp8_gemm_nt_contiguous(const void* a, const float* sfa, int64_t ld_sfa, const void* b,
                                              const float* sfb, void* d, dg_dtype d_dtype,
                                              const int32_t* m_indices, int m_total, int n, int k,
                                              int num_groups, hipStream_t stream) {
  return contiguous_impl(a, sfa, ld_sfa, b, sfb, d, d_dtype, m_indices, m_total, n, k, num_groups, false, stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_masked(const void* a, const float* sfa, int64_t ld_sfa, const void* b,
                                          const float* sfb, void* d, dg_dtype d_dtype, const int32_t* masked_m,
                                          int num_groups, int m_max, int n, int k, int expected_m,
                                          hipStream_t stream) {
  return masked_impl(a, sfa, ld_sfa, b, sfb, d, d_dtype, masked_m, num_groups, m_max, n, k, expected_m, false,
                     stream);
}

dg_status dg_fp8_gemm_nt_ue8m0(const void* a, int64_t lda, const int32_t* sfa, int64_t ld_sfa, const void* b,
                               int64_t ldb, const int32_t* sfb, const void* c, int64_t ldc, void* d, int64_t ldd,
                               dg_dtype d_dtype, int m, int n, int k, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  return dense_impl(a, lda, sfa, ld_sfa, b, ldb, sfb, c, ldc, d, ldd, d_dtype, m, n, k, true, workspace,
                    workspace_bytes, stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(const void* a, const int32_t* sfa, int64_t ld_sfa,
                                                    const void* b, const int32_t* sfb, void* d, dg_dtype d_dtype,
                                                    const int32_t* m_indices, int m_total, int n, int k,
                                                    int num_groups, hipStream_t stream) {
  return contiguous_impl(a, sfa, ld_sfa, b, sfb, d, d_dtype, m_indices, m_total, n, k, num_groups, true, stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_masked_ue8m0(const void* a, const int32_t* sfa, int64_t ld_sfa, const void* b,
                                                const int32_t* sfb, void* d, dg_dtype d_dtype,
                                                const int32_t* masked_m, int num_groups, int m_max, int n, int k,
                                                int expected_m, hipStream_t stream) {
  return masked_impl(a, sfa, ld_sfa, b, sfb, d, d_dtype, masked_m, num_groups, m_max, n, k, expected_m, true,
                     stream);
}

dg_status dg_k_grouped_fp8_gemm_nt_contiguous(const void* a, const float* sfa, int64_t ld_sfa, const void* b,
                                              const float* sfb, const float* c, float* d, const int32_t* ks,
                                              int num_groups, int m, int n, int k_total, hipStream_t stream) {
  return k_grouped_impl(a, sfa, ld_sfa, b, sfb, c, d, ks, num_groups, m, n, k_total, false, stream);
}

dg_status dg_k_grouped_fp8_gemm_nt_contiguous_ue8m0(const void* a, const int32_t* sfa, int64_t ld_sfa,
                                                    const void* b, const int32_t* sfb, const float* c, float* d,
                                                    const int32_t* ks, int num_groups, int m, int n, int k_total,
                                                    hipStream_t stream) {
  return k_grouped_impl(a, sfa, ld_sfa, b, sfb, c, d, ks, num_groups, m, n, k_total, true, stream);
}

dg_status dg_wgrad_fp8_gemm_nt(const void* a, int64_t lda, const float* sfa, int64_t ld_sfa, const void* b,
                               int64_t ldb, const float* sfb, float* d, int64_t ldd, int m, int n, int k,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return dense_impl(a, lda, sfa, ld_sfa, b, ldb, sfb, d, ldd, d, ldd, DG_DTYPE_FP32, m, n, k, false, workspace,
                    workspace_bytes, stream);
}

dg_status dg_k_grouped_wgrad_fp8_gemm_nt(const void* a, const float* sfa, int64_t ld_sfa, const void* b,
                                         const float* sfb, float* d, const int32_t* ks, int num_groups, int m,
                                         int n, int k_total, hipStream_t stream) {
  return k_grouped_impl(a, sfa, ld_sfa, b, sfb, d, d, ks, num_groups, m, n, k_total, false, stream);
}

dg_status dg_k_grouped_wgrad_fp8_gemm_nt_ue8m0(const void* a, const int32_t* sfa, int64_t ld_sfa, const void* b,
                                               const int32_t* sfb, float* d, const int32_t* ks, int num_groups,
                                               int m, int n, int k_total, hipStream_t stream) {
  return k_grouped_impl(a, sfa, ld_sfa, b, sfb, d, d, ks, num_groups, m, n, k_total, true, stream);
}

int dg_get_mk_alignment_for_contiguous_layout(void) { return kAlignM; }

int64_t dg_get_sf_aligned_size(int64_t mn) { return mn < 0 ? -1 : (mn + 3) / 4 * 4; }

dg_status dg_set_num_cus(int num_cus) {
  if (num_cus < 0) return DG_ERROR_INVALID_VALUE;
  read_env();
  g_num_cus.store(num_cus);
  return DG_SUCCESS;
}

int dg_get_num_cus(void) {
  read_env();
  const int cap = g_num_cus.load();
  int dev = 0, total = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&total, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || total <= 0) {
    (void)hipGetLastError();
    return cap;  // no device: the cap (0 = uncapped)
  }
  return (cap > 0 && cap < total) ? cap : total;
}

dg_status dg_internal_dense_plan(int m, int n, int k, int cus, int* bm, int* bn, int* splits, int* slabs_per_split,
                                 size_t* ws_bytes) {
  if (m <= 0 || n <= 0 || k <= 0 || k % 128 != 0 || cus <= 0) return DG_ERROR_INVALID_VALUE;
  if (bm == nullptr || bn == nullptr || splits == nullptr || slabs_per_split == nullptr || ws_bytes == nullptr)
    return DG_ERROR_INVALID_VALUE;
  const DensePlan pl = plan_dense_for(m, n, k, cus);
  *bm = pl.cfg.bm;
  *bn = pl.cfg.bn;
  *splits = pl.splits;
  *slabs_per_split = pl.slabs_per_split;
  *ws_bytes = pl.ws_bytes;
  return DG_SUCCESS;
}

dg_status dg_internal_set_tile_n(int tile_n) {
  if (tile_n != 0 && tile_n != 256 && tile_n != 224 && tile_n != 160) return DG_ERROR_INVALID_VALUE;
  g_tile_n.store(tile_n);
  return DG_SUCCESS;
}

const char* dg_status_string(dg_status s) {
  switch (s) {
    case DG_SUCCESS: return "DG_SUCCESS";
    case DG_ERROR_INVALID_VALUE: return "DG_ERROR_INVALID_VALUE: invalid argument (pointer, alignment, stride, size or dtype)";
    case DG_ERROR_NOT_SUPPORTED: return "DG_ERROR_NOT_SUPPORTED: shape not supported (K % 128 != 0 or contiguous M % 128 != 0)";
    case DG_ERROR_LAUNCH_FAILED: return "DG_ERROR_LAUNCH_FAILED: a HIP call failed";
    case DG_ERROR_SCRATCH_LIMIT:
      return "DG_ERROR_SCRATCH_LIMIT: the call needs more split-K scratch than the allocation-free entry point "
             "holds (16 MiB of partial tiles); use dg_fp8_gemm_nt with a workspace";
    case DG_ERROR_WORKSPACE:
      return "DG_ERROR_WORKSPACE: the split-K workspace is missing, not 256-byte aligned or smaller than "
             "dg_get_workspace_size(m, n, k)";
  }
  return "DG_UNKNOWN_STATUS";
}

const char* dg_last_hip_error(void) { return dg::g_last_hip_error; }

}  // extern "C"
