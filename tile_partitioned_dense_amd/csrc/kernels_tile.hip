// kernels_tile.hip -- instances of the tile kernel for one configuration,
// selected at compile time with -DTG_TILE_CONFIG=<index into kTileConfigs>.
#include "launch.hpp"

#ifndef TG_TILE_CONFIG
#error "TG_TILE_CONFIG must name a tile configuration index"
#endif

namespace tg {

template <int CFG>
hipError_t launch_tile(const TileArgs& a, int64_t grid_wgs, const Variant& v, hipStream_t stream) {
  constexpr TileConfig c = kTileConfigs[CFG];
  const dim3 grid((unsigned)grid_wgs);
  const dim3 block(c.wm * c.wn * 64);
#define TG_TILE_FN(BC, OB, DB) \
  reinterpret_cast<const void*>(&tile_gemm_kernel<c.bm, c.bn, c.wm, c.wn, c.stages, BC, OB, DB>)
  const void* fn;
  if (v.b_col_major) {
    if (v.out_bf16) fn = v.debug ? TG_TILE_FN(true, true, true) : TG_TILE_FN(true, true, false);
    else fn = v.debug ? TG_TILE_FN(true, false, true) : TG_TILE_FN(true, false, false);
  } else {
    if (v.out_bf16) fn = v.debug ? TG_TILE_FN(false, true, true) : TG_TILE_FN(false, true, false);
    else fn = v.debug ? TG_TILE_FN(false, false, true) : TG_TILE_FN(false, false, false);
  }
#undef TG_TILE_FN
  return launch_raw(fn, grid, block, a, stream);
}

template hipError_t launch_tile<TG_TILE_CONFIG>(const TileArgs&, int64_t, const Variant&, hipStream_t);

}  // namespace tg
