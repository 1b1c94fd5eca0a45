// kernels_tile.hip -- instances of the tile kernel for one configuration,
// selected at compile time with -DTG_TILE_CONFIG=<index into kTileConfigs>.
#include "launch.hpp"

#ifndef TG_TILE_CONFIG
#error "TG_TILE_CONFIG must name a tile configuration index"
#endif

namespace tg {

// The kernel instance of configuration CFG: the tile kernel (on 32x32x16 or
// 16x16x32 MFMA blocks), the K-split kernel for configurations whose waves
// share K, or the stream kernel (column-major B only; NULL for a row-major B).
template <int CFG, bool BC, bool OB, bool DB>
const void* tile_fn() {
  constexpr TileConfig c = kTileConfigs[CFG];
  if constexpr (c.sb > 0) {
    if constexpr (BC)
      return reinterpret_cast<const void*>(&stream_gemm_kernel<c.bm, c.bn, c.sb, c.stages, c.ks, OB, DB>);
    else
      return nullptr;
  } else if constexpr (c.ks > 1)
    return reinterpret_cast<const void*>(&ksplit_gemm_kernel<c.bm, c.bn, c.ks, c.stages, BC, OB, DB>);
  else if constexpr (c.mi == 16 && c.bk == 64)
    return reinterpret_cast<const void*>(&tile64_gemm_kernel<c.bm, c.bn, c.wm, c.wn, BC, OB, DB>);
  else if constexpr (c.mi == 16)
    return reinterpret_cast<const void*>(&tile16_gemm_kernel<c.bm, c.bn, c.wm, c.wn, c.stages, BC, OB, DB>);
  else
    return reinterpret_cast<const void*>(&tile_gemm_kernel<c.bm, c.bn, c.wm, c.wn, c.stages, BC, OB, DB>);
}

template <int CFG>
hipError_t launch_tile(const TileArgs& a, int64_t grid_wgs, const Variant& v, hipStream_t stream) {
  constexpr TileConfig c = kTileConfigs[CFG];
  const dim3 grid((unsigned)grid_wgs);
  const dim3 block(c.wm * c.wn * c.ks * 64);
  const void* fn;
  if (v.b_col_major) {
    if (v.out_bf16) fn = v.debug ? tile_fn<CFG, true, true, true>() : tile_fn<CFG, true, true, false>();
    else fn = v.debug ? tile_fn<CFG, true, false, true>() : tile_fn<CFG, true, false, false>();
  } else {
    if (v.out_bf16) fn = v.debug ? tile_fn<CFG, false, true, true>() : tile_fn<CFG, false, true, false>();
    else fn = v.debug ? tile_fn<CFG, false, false, true>() : tile_fn<CFG, false, false, false>();
  }
  if (!fn) return hipErrorInvalidValue;
  return launch_raw(fn, grid, block, a, stream);
}

template hipError_t launch_tile<TG_TILE_CONFIG>(const TileArgs&, int64_t, const Variant&, hipStream_t);

}  // namespace tg
