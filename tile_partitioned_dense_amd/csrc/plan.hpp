// plan.hpp -- output-tile partitioner and launch planner.
//
// The output C is split into disjoint tiles before launch and each tile is
// exclusively owned by one workgroup: the host-side partition that "GPU speed,
// without leaving Rust's safety model" describes in "Ownership crosses the
// launch boundary" (a mutable output partitioned into exclusive
// sub-tensors, inputs broadcast as shared views) and "Disjointness outside.
// Ordering inside." (the owned sub-tensor is the destination; no program
// picks a store index of its own).
//
// tile_of() is compiled for both host and device: the kernels call it to find
// their owned tile, and the host-side tests call the very same function to
// check that it is a bijection onto the tile grid.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define TG_HD __host__ __device__ __forceinline__
#else
#define TG_HD inline
#endif

namespace tg {

constexpr int kBK = 32;            // K slab staged per step in the tile kernel
constexpr int kSkinnyMaxM = 16;    // M at or below this takes the skinny kernel; above
                                   // it the K-split tile kernel measured faster
constexpr int kSkinnyWaves = 8;    // waves per skinny workgroup, splitting K
constexpr int kXcds = 8;           // MI355X: 8 accelerator dies share one dispatcher

// Tile-kernel configurations compiled into the library. `eff` (and `eff1`
// for a workgroup alone on its compute unit) is the throughput a compute
// unit sustains on this configuration relative to configuration 7, measured
// with random bf16 data in interleaved cold-cache runs; the planner uses it
// only to rank configurations for a shape. Eight-wave configurations put two
// waves on each SIMD, so one wave's LDS reads, loads and barrier waits overlap
// the other's MFMAs. K-split configurations (ks > 1) serve outputs with few
// or small tiles and a long K.
struct TileConfig {
  int bm, bn;   // owned tile
  int wm, wn;   // wave grid inside the workgroup (each wave owns (bm/wm) x (bn/wn))
  int stages;   // depth of the LDS ring of 32-wide K slabs (per wave when ks > 1)
  float eff;    // rate with `occ` workgroups sharing each compute unit
  int ks = 1;   // > 1: that many waves each take the whole tile over a share of
                // K and combine in a fixed tree (ksplit_kernel.hpp)
  float eff1 = 0.0f;  // rate of a workgroup alone on its compute unit (0: = eff)
  int occ = 1;        // workgroups that fit on one compute unit at once
  int sb = 0;         // > 0: the stream kernel (stream_kernel.hpp, column-major B
                      // only) with stages of sb bytes of K per row
  int mi = 32;        // MFMA block: 32 (32x32x16, tile_kernel.hpp) or 16
                      // (16x16x32, tile16_kernel.hpp)
  int bk = 32;        // K per slab: 32, or 64 (tile64_kernel.hpp: 16x16x32
                      // blocks, two stages of 128-byte rows)
};

// Rate of configuration c when each compute unit has `per_cu` of its tiles:
// small-LDS configurations hide load latency only with several workgroups on
// one compute unit (alone, a 64 x 64 tile's four waves wait on every slab).
inline double tile_eff(const TileConfig& c, int64_t per_cu) {
  const double e1 = c.eff1 > 0.0f ? c.eff1 : c.eff;
  if (c.occ <= 1 || per_cu <= 1) return per_cu <= 1 ? e1 : c.eff;
  const int64_t n = per_cu < c.occ ? per_cu : c.occ;
  return e1 + (c.eff - e1) * (double)(n - 1) / (double)(c.occ - 1);
}

constexpr int kNumTileConfigs = 29;
constexpr TileConfig kTileConfigs[kNumTileConfigs] = {
    {256, 256, 2, 2, 4, 0.94f},  // 0: 4 waves of 128x128
    {256, 224, 4, 1, 5, 0.85f},  // 1: 4 waves of 64x224
    {256, 160, 4, 1, 5, 0.81f},  // 2: 4 waves of 64x160
    {128, 256, 2, 2, 5, 0.85f},  // 3: 4 waves of 64x128
    {256, 128, 2, 2, 5, 0.78f},  // 4: 4 waves of 128x64
    {128, 128, 2, 2, 4, 0.81f, 1, 0.59f, 2},  // 5: 4 waves of 64x64
    {64, 64, 2, 2, 4, 0.46f, 1, 0.17f, 4},    // 6: 4 waves of 32x32
    {256, 256, 2, 4, 4, 1.00f},  // 7: 8 waves of 128x64
    {256, 256, 4, 2, 4, 0.99f},  // 8: 8 waves of 64x128
    {256, 224, 8, 1, 5, 0.85f},  // 9: 8 waves of 32x224
    {256, 160, 8, 1, 5, 0.82f},  // 10: 8 waves of 32x160
    {64, 64, 1, 1, 4, 0.28f, 4},    // 11: 4 waves, each 64x64 over a quarter of K
    {64, 128, 1, 1, 3, 0.42f, 4},   // 12: 4 waves, each 64x128 over a quarter of K
    {128, 64, 1, 1, 3, 0.39f, 4},   // 13: 4 waves, each 128x64 over a quarter of K
    // 14-16: stream, 3 stages, two waves per 32-column block, each taking
    // half of every stage's K: 32 rows x 64 columns with stages of 512 bytes
    // per row (up to 32 rows), 64 x 128 with 256 bytes (33 to 64 rows), and
    // 64 x 64 with 256 bytes (33 to 64 rows with few columns)
    {32, 64, 1, 2, 3, 0.0f, 2, 0.0f, 1, 512},
    {64, 128, 1, 4, 3, 0.0f, 2, 0.0f, 1, 256},
    {64, 64, 1, 2, 3, 0.0f, 2, 0.0f, 1, 256},
    // 17-23: the tile kernel on 16x16x32 blocks (two waves per SIMD issue it
    // at close to the full MFMA rate, the 32x32x16 form at about 60%)
    {256, 256, 2, 4, 4, 1.09f, 1, 0.0f, 1, 0, 16},  // 17: 8 waves of 128x64
    {256, 256, 2, 4, 5, 1.08f, 1, 0.0f, 1, 0, 16},  // 18: the same with 5 stages
    {256, 160, 4, 2, 4, 0.83f, 1, 0.0f, 1, 0, 16},  // 19: 8 waves of 64x80
    {128, 256, 2, 4, 5, 0.80f, 1, 0.0f, 1, 0, 16},  // 20: 8 waves of 64x64
    {256, 128, 4, 2, 5, 0.77f, 1, 0.0f, 1, 0, 16},  // 21: 8 waves of 64x64
    // 22-23: one wave per SIMD on 16x16 blocks: the 128-wide wave tiles read a
    // third less from LDS; their 256 accumulators fill the accumulation
    // registers, where the MFMAs are written out with the accumulator tied in
    // place (tile16_kernel.hpp, mma16)
    {256, 256, 2, 2, 4, 1.05f, 1, 0.94f, 1, 0, 16},  // 22: 4 waves of 128x128
    {256, 160, 2, 2, 4, 0.84f, 1, 0.0f, 1, 0, 16},   // 23: 4 waves of 128x80
    // 24-25: 16x16x32 blocks with 64-deep slabs (two stages of 128-byte rows;
    // each load instruction moves whole 128-byte lines)
    {256, 256, 2, 4, 2, 0.01f, 1, 0.0f, 1, 0, 16, 64},  // 24: 8 waves of 128x64
    {256, 160, 4, 2, 2, 0.01f, 1, 0.0f, 1, 0, 16, 64},  // 25: 8 waves of 64x80
    // 26-27: one wave per SIMD, 64-deep slabs, accumulators tied in place
    // (its own K-loop order, tile64_kernel.hpp); with a single 256 x 256 tile
    // per CU level with configuration 17, which keeps those shapes
    {256, 256, 2, 2, 2, 1.19f, 1, 1.08f, 1, 0, 16, 64},  // 26: 4 waves of 128x128
    {256, 160, 2, 2, 2, 1.04f, 1, 1.05f, 1, 0, 16, 64},  // 27: 4 waves of 128x80
    // 28: 256 x 224 (a 7168-wide output splits into 32 columns of tiles, 1024
    // tiles fill four rounds of all 256 compute units where 256 x 256 tiles
    // leave 32 of them idle)
    {256, 224, 2, 2, 2, 1.15f, 1, 1.07f, 1, 0, 16, 64},  // 28: 4 waves of 128x112
};
constexpr int kStreamConfig = 14;      // the planner's stream configuration up to 32 rows,
constexpr int kStreamConfig64 = 15;    // from 33 to 64 rows,
constexpr int kStreamConfig64n = 16;   // and from 33 to 64 rows with few columns
constexpr int kStreamMaxM = 64;      // column-major B, even K and M at or below this: stream kernel

// Skinny-kernel configurations: T output columns per lane (16*T per
// workgroup) and MG groups of 16 rows.
struct SkinnyConfig {
  int t, mg;
};
constexpr int kNumSkinnyConfigs = 6;
constexpr SkinnyConfig kSkinnyConfigs[kNumSkinnyConfigs] = {
    {4, 1}, {8, 1}, {4, 2}, {8, 2}, {4, 4}, {8, 4},
};

// MX configurations: the tile kernel (mx_kernel.hpp; `eff` ranks them as in
// the bf16 table) and, with `sb` set, the few-row streaming kernel
// (mx_stream_kernel.hpp: one 16- or 32-row block, sb bytes of K per row and
// stage, one wave per 32 columns), which the planner takes for short outputs.
struct MxConfig {
  int bm, bn, wm, wn, stages;
  float eff;
  int sb = 0;  // stream kernel: bytes of K per row and stage; 0: tile kernel
  int ks = 1;  // stream kernel: waves per 32-column block (each a share of every stage's K)
  int rb = 64;  // tile kernel: bytes per row and stage (128: two slabs, mx128_kernel.hpp)
  int mi = 32;  // tile kernel: MFMA block, 32 (32x32x64) or 16 (16x16x128, mx16_kernel.hpp;
                // K a multiple of 128)
  float eff4 = 0.0f;  // tile kernel: rate with E2M1 elements (0: eff)
};
constexpr int kNumMxConfigs = 8;
constexpr MxConfig kMxConfigs[kNumMxConfigs] = {
    {256, 256, 2, 2, 4, 1.00f},  // 0: 4 waves of 128x128
    {128, 128, 2, 2, 4, 0.70f},  // 1: 4 waves of 64x64
    {64, 128, 2, 2, 12, 0.50f},  // 2: 4 waves of 32x64, 12 stages: few rows, weight streaming
    // 3, 4: stream, 32 or 64 rows x 128 columns, 3 stages of 256 bytes, two
    // waves per 32-column block, each taking half of every stage's slabs
    {32, 128, 1, 4, 3, 0.0f, 256, 2},
    {64, 128, 1, 4, 3, 0.0f, 256, 2},
    // 5: stream, 32 x 64 with stages of 512 bytes: twice the workgroups of
    // configuration 3, for outputs with few columns
    {32, 64, 1, 2, 3, 0.0f, 512, 2},
    // 6: 4 waves of 128x128, 128-byte rows (two slabs per stage, two stages;
    // 1.09 times configuration 0 on the MXFP8 MLP shard, 1.06 on MXFP4,
    // interleaved in one process)
    {256, 256, 2, 2, 2, 1.09f, 0, 1, 128, 32, 1.06f},
    // 7: 4 waves of 128x112 on 16x16x128 blocks, 128-byte rows (one E4M3 or
    // two E2M1 K steps per stage, two stages): 256 x 224 tiles fill all
    // compute units on a 7168-wide output. Per compute unit 0.92 times
    // configuration 6 with E4M3 and 0.91 times with E2M1; the MLP shard's
    // launch is 4% shorter (E4M3) and 1-6% shorter (E2M1), interleaved in one
    // process.
    {256, 224, 2, 2, 2, 1.00f, 0, 1, 128, 16, 0.96f},
};
constexpr int kMxBK = 64;          // bytes of K per row in one slab of the MX tile kernel
constexpr int kMxStreamMaxM = 64;  // M at or below this takes the stream kernel

// Owned-tile map parameters (kernel argument; plain data).
struct TileMap {
  int32_t tiles_m, tiles_n;
  int32_t group_m;  // tile rows per raster group
  int32_t xcds;     // dispatch remap width; 1 = identity
};

TG_HD int32_t tg_min(int32_t a, int32_t b) { return a < b ? a : b; }

// Workgroup id -> owned tile (tm, tn). A bijection from [0, tiles_m*tiles_n)
// onto the tile grid, composed of two bijections:
//  1. dispatch remap: consecutive workgroup ids land on different XCDs
//     (round-robin), so give XCD x one contiguous range of tile indices and
//     let its workgroups walk that range in dispatch order; tiles that run
//     at the same time on one XCD then share its L2;
//  2. grouped raster: group_m tile rows at a time, walking down the rows of a
//     group before moving to the next column, so co-running tiles reuse the
//     same A row panels and B column panels.
TG_HD void tile_of(const TileMap& mp, int32_t wg, int32_t& tm, int32_t& tn) {
  const int32_t T = mp.tiles_m * mp.tiles_n;
  int32_t t = wg;
  if (mp.xcds > 1) {
    const int32_t q = T / mp.xcds, r = T - (T / mp.xcds) * mp.xcds;
    const int32_t x = wg % mp.xcds, i = wg / mp.xcds;
    t = x * q + tg_min(x, r) + i;
  }
  const int32_t per_group = mp.group_m * mp.tiles_n;
  const int32_t g = t / per_group;
  const int32_t first_m = g * mp.group_m;
  const int32_t gsz = tg_min(mp.tiles_m - first_m, mp.group_m);
  const int32_t local = t - g * per_group;
  tm = first_m + local % gsz;
  tn = local / gsz;
}

struct Plan {
  int variant;  // 0 none, 1 tile, 2 skinny, 3 MXFP8 tile
  int config;
  int bm, bn, bk, threads, lds_bytes;
  TileMap map;
  int k_split;
  int64_t tiles;  // owned tiles
  int64_t grid;   // workgroups launched
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int tile_lds_bytes(const TileConfig& c) {
  if (c.sb) return c.stages * (c.bm + c.bn) * c.sb;
  const int ring = c.ks * c.stages * (c.bm + c.bn) * c.bk * 2;
  const int tree = (c.ks / 2) * c.bm * c.bn * 4;
  return ring > tree ? ring : tree;
}
inline int skinny_lds_bytes(const SkinnyConfig& c) {
  return (kSkinnyWaves / 2) * c.mg * c.t * 64 * 16;
}

// Raster group height: enough tile rows that the tiles co-running on one XCD
// (32 compute units) form a roughly square block of the tile grid.
inline int32_t pick_group_m(int32_t tiles_m, int32_t tiles_n) {
  // 8 rows for narrow grids; 8 also for wide ones (at 32 x 28 tiles of
  // 256 x 256, 8 rows measured 2-3% faster than 4 and 16 rows 10% slower)
  int32_t g = 4;
  if (tiles_n < 8 || tiles_n >= 16) g = 8;
  if (g > tiles_m) g = tiles_m;
  return g < 1 ? 1 : g;
}

// Workgroups for `tiles` tiles on `cu_count` compute units: as many as one
// round of tiles needs when the tiles fit in one round; otherwise the tiles
// are shared out evenly over ceil(tiles / cu_count) rounds, each workgroup
// taking tiles t, t + grid, t + 2 grid, ... Every workgroup then runs the same
// number of tiles (give or take one), instead of a last round that leaves
// part of the chip idle, and the idle units' power budget goes to the busy
// ones. The count is rounded up to a multiple of the XCD count where that
// still fits the compute units, so all tiles of a workgroup stay on its XCD
// (t and t + grid share t % kXcds).
inline int64_t persistent_grid(int64_t tiles, int cu_count) {
  if (tiles <= cu_count) return tiles;
  const int64_t rounds = ceil_div(tiles, cu_count);
  const int64_t g0 = ceil_div(tiles, rounds);
  const int64_t g = ceil_div(g0, kXcds) * kXcds;
  return g <= cu_count ? g : g0;
}

// The launch geometry of one configuration for an M x N output.
inline Plan plan_for(int variant, int config, int64_t M, int64_t N, int cu_count) {
  Plan p{};
  p.bk = kBK;
  p.map.xcds = 1;
  p.variant = variant;
  p.config = config;
  if (variant == 2) {
    const SkinnyConfig& c = kSkinnyConfigs[config];
    p.bm = 16 * c.mg;
    p.bn = 16 * c.t;
    p.threads = kSkinnyWaves * 64;
    p.lds_bytes = skinny_lds_bytes(c);
    p.k_split = kSkinnyWaves;
    p.map.tiles_m = 1;
    p.map.tiles_n = (int32_t)ceil_div(N, p.bn);
    p.map.group_m = 1;
    p.tiles = p.map.tiles_n;
    p.grid = p.tiles;
  } else if (variant == 1) {
    const TileConfig& c = kTileConfigs[config];
    p.bm = c.bm;
    p.bn = c.bn;
    p.threads = c.wm * c.wn * c.ks * 64;
    p.lds_bytes = tile_lds_bytes(c);
    p.bk = c.sb ? c.sb / 2 : c.bk;
    p.k_split = c.ks;
    p.map.tiles_m = (int32_t)ceil_div(M, c.bm);
    p.map.tiles_n = (int32_t)ceil_div(N, c.bn);
    p.map.group_m = pick_group_m(p.map.tiles_m, p.map.tiles_n);
    p.map.xcds = kXcds;
    p.tiles = (int64_t)ceil_div(M, c.bm) * ceil_div(N, c.bn);
    p.grid = persistent_grid(p.tiles, cu_count);
  }
  return p;
}

// The launch geometry of MX configuration `config` for an M x N output.
inline Plan plan_for_mx(int config, int64_t M, int64_t N, int cu_count) {
  Plan p{};
  const MxConfig& c = kMxConfigs[config];
  p.variant = 3;
  p.config = config;
  p.bm = c.bm;
  p.bn = c.bn;
  p.bk = c.sb ? c.sb : c.rb;
  p.threads = c.wm * c.wn * c.ks * 64;
  p.lds_bytes = c.stages * (c.bm + c.bn) * p.bk;
  p.k_split = 1;
  p.map.tiles_m = (int32_t)ceil_div(M, c.bm);
  p.map.tiles_n = (int32_t)ceil_div(N, c.bn);
  p.map.group_m = pick_group_m(p.map.tiles_m, p.map.tiles_n);
  p.map.xcds = kXcds;
  p.tiles = (int64_t)p.map.tiles_m * p.map.tiles_n;
  p.grid = persistent_grid(p.tiles, cu_count);
  return p;
}

// MX plan: outputs of at most kMxStreamMaxM rows stream B through the
// stream kernel (one tile row of 32 or 64 rows); otherwise the tile-kernel configuration
// minimising (tiles on the busiest CU) x (tile area) / rate, as for the bf16
// tile kernel, with the rate of the element format (fp4: E2M1).
inline Plan make_plan_mx(int64_t M, int64_t N, int64_t K, bool fp4, int cu_count) {
  if (M <= 0 || N <= 0) return plan_for(0, 0, M, N, cu_count);
  if (M <= kMxStreamMaxM) {
    // up to 32 rows: 128-column tiles, or 64-column ones when those would
    // leave more than half of the compute units without a tile
    const int c = M > 32 ? 4 : (2 * ceil_div(N, 128) < cu_count ? 5 : 3);
    return plan_for_mx(c, M, N, cu_count);
  }
  int best = 0;
  double best_cost = 0.0;
  for (int i = 0; i < kNumMxConfigs; ++i) {
    const MxConfig& c = kMxConfigs[i];
    if (c.sb || (c.mi == 16 && K % 128 != 0)) continue;
    const int64_t per_cu = ceil_div(ceil_div(M, c.bm) * ceil_div(N, c.bn), cu_count);
    const float eff = (fp4 && c.eff4 > 0.0f) ? c.eff4 : c.eff;
    const double cost = (double)per_cu * c.bm * c.bn / eff;
    if (i == 0 || cost < best_cost * 0.999) {
      best = i;
      best_cost = cost;
    }
  }
  return plan_for_mx(best, M, N, cu_count);
}

// Pure function of (M, N, K, B layout, CU count). The output type is not an
// input, so fp32 and bf16 outputs of one shape share kernel, tile and K order.
inline Plan make_plan(int64_t M, int64_t N, int64_t K, bool b_col_major, int cu_count) {
  if (M <= 0 || N <= 0) return plan_for(0, 0, M, N, cu_count);
  // (odd K: the stream kernel's loads of whole dwords would drop the value
  // K - 1 of each operand's last row, so those shapes stay on the others)
  if (b_col_major && M <= kStreamMaxM && K % 2 == 0)
    return plan_for(1, M <= 32 ? kStreamConfig
                               : (2 * ceil_div(N, 128) < cu_count ? kStreamConfig64n : kStreamConfig64),
                    M, N, cu_count);
  if (M <= kSkinnyMaxM) {
    const int mg = (int)ceil_div(M, 16);
    const int mgp = mg <= 1 ? 1 : (mg <= 2 ? 2 : 4);
    // wide column stripes (longer contiguous row segments) unless that
    // leaves fewer than half as many workgroups as compute units
    const int t = (2 * ceil_div(N, 128) >= cu_count) ? 8 : 4;
    int idx = 0;
    for (int i = 0; i < kNumSkinnyConfigs; ++i)
      if (kSkinnyConfigs[i].t == t && kSkinnyConfigs[i].mg == mgp) idx = i;
    return plan_for(2, idx, M, N, cu_count);
  }
  // Tile kernel: minimise (tiles on the busiest CU) x (tile area) / rate.
  int best = 0;
  double best_cost = 0.0;
  for (int i = 0; i < kNumTileConfigs; ++i) {
    const TileConfig& c = kTileConfigs[i];
    if (c.sb) continue;
    const int64_t tiles = ceil_div(M, c.bm) * ceil_div(N, c.bn);
    const int64_t per_cu = ceil_div(tiles, cu_count);
    const double cost = (double)per_cu * c.bm * c.bn / tile_eff(c, per_cu);
    if (i == 0 || cost < best_cost * 0.999) {
      best = i;
      best_cost = cost;
    }
  }
  return plan_for(1, best, M, N, cu_count);
}

}  // namespace tg
