// kernels_skinny.hip -- instances of the skinny kernel for one configuration,
// selected at compile time with -DTG_SKINNY_CONFIG=<index into kSkinnyConfigs>.
#include "launch.hpp"

#ifndef TG_SKINNY_CONFIG
#error "TG_SKINNY_CONFIG must name a skinny configuration index"
#endif

namespace tg {

constexpr int kSkinnyUnroll = 2;  // 32-k blocks whose loads are issued together

template <int CFG>
hipError_t launch_skinny(const SkinnyArgs& a, int64_t grid_n, const Variant& v, hipStream_t stream) {
  constexpr SkinnyConfig c = kSkinnyConfigs[CFG];
  const dim3 grid((unsigned)grid_n);
  const dim3 block(kSkinnyWaves * 64);
#define TG_SK_FN(BC, OB, DB)                                                                  \
  reinterpret_cast<const void*>(                                                              \
      &skinny_gemm_kernel<c.t, kSkinnyWaves, c.mg, kSkinnyUnroll, BC, OB, DB>)
  const void* fn;
  if (v.b_col_major) {
    if (v.out_bf16) fn = v.debug ? TG_SK_FN(true, true, true) : TG_SK_FN(true, true, false);
    else fn = v.debug ? TG_SK_FN(true, false, true) : TG_SK_FN(true, false, false);
  } else {
    if (v.out_bf16) fn = v.debug ? TG_SK_FN(false, true, true) : TG_SK_FN(false, true, false);
    else fn = v.debug ? TG_SK_FN(false, false, true) : TG_SK_FN(false, false, false);
  }
#undef TG_SK_FN
  return launch_raw(fn, grid, block, a, stream);
}

template hipError_t launch_skinny<TG_SKINNY_CONFIG>(const SkinnyArgs&, int64_t, const Variant&,
                                                   hipStream_t);

}  // namespace tg
