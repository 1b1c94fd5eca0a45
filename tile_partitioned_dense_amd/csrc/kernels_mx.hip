// kernels_mx.hip -- instances of the MX kernels (tile or stream) for one
// configuration, selected at compile time with -DTG_MX_CONFIG=<index into
// kMxConfigs>.
#include "launch.hpp"

#ifndef TG_MX_CONFIG
#error "TG_MX_CONFIG must name an MX configuration index"
#endif

namespace tg {

template <int CFG, int FMT, bool OB, bool DB>
const void* mx_fn() {
  constexpr MxConfig c = kMxConfigs[CFG];
  if constexpr (c.sb > 0)
    return reinterpret_cast<const void*>(&mx_stream_kernel<c.bm, c.bn, c.sb, c.stages, c.ks, FMT, OB, DB>);
  else if constexpr (c.mi == 16)
    return reinterpret_cast<const void*>(&mx16_gemm_kernel<c.bm, c.bn, c.wm, c.wn, FMT, OB, DB>);
  else if constexpr (c.rb == 128)
    return reinterpret_cast<const void*>(&mx128_gemm_kernel<c.bm, c.bn, c.wm, c.wn, FMT, OB, DB>);
  else
    return reinterpret_cast<const void*>(&mx_gemm_kernel<c.bm, c.bn, c.wm, c.wn, c.stages, FMT, OB, DB>);
}

template <int CFG, int FMT>
const void* mx_fn_out(const Variant& v) {
  if (v.out_bf16) return v.debug ? mx_fn<CFG, FMT, true, true>() : mx_fn<CFG, FMT, true, false>();
  return v.debug ? mx_fn<CFG, FMT, false, true>() : mx_fn<CFG, FMT, false, false>();
}

template <int CFG>
hipError_t launch_mx(const MxArgs& a, int fmt, int64_t grid_wgs, const Variant& v,
                     hipStream_t stream) {
  constexpr MxConfig c = kMxConfigs[CFG];
  const dim3 grid((unsigned)grid_wgs);
  const dim3 block(c.wm * c.wn * c.ks * 64);
  const void* fn = fmt == kMxE2M1 ? mx_fn_out<CFG, kMxE2M1>(v) : mx_fn_out<CFG, kMxE4M3>(v);
  return launch_raw(fn, grid, block, a, stream);
}

template hipError_t launch_mx<TG_MX_CONFIG>(const MxArgs&, int, int64_t, const Variant&, hipStream_t);

}  // namespace tg
