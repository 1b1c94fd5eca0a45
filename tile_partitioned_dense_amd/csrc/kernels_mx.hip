// kernels_mx.hip -- instances of the MXFP8 tile kernel for one configuration,
// selected at compile time with -DTG_MX_CONFIG=<index into kMxConfigs>.
#include "launch.hpp"

#ifndef TG_MX_CONFIG
#error "TG_MX_CONFIG must name an MX configuration index"
#endif

namespace tg {

template <int CFG, bool OB, bool DB>
const void* mx_fn() {
  constexpr MxConfig c = kMxConfigs[CFG];
  return reinterpret_cast<const void*>(&mx_gemm_kernel<c.bm, c.bn, c.wm, c.wn, c.stages, OB, DB>);
}

template <int CFG>
hipError_t launch_mx(const MxArgs& a, int64_t grid_wgs, const Variant& v, hipStream_t stream) {
  constexpr MxConfig c = kMxConfigs[CFG];
  const dim3 grid((unsigned)grid_wgs);
  const dim3 block(c.wm * c.wn * 64);
  const void* fn;
  if (v.out_bf16) fn = v.debug ? mx_fn<CFG, true, true>() : mx_fn<CFG, true, false>();
  else fn = v.debug ? mx_fn<CFG, false, true>() : mx_fn<CFG, false, false>();
  return launch_raw(fn, grid, block, a, stream);
}

template hipError_t launch_mx<TG_MX_CONFIG>(const MxArgs&, int64_t, const Variant&, hipStream_t);

}  // namespace tg
