// launch.hpp -- launchers for the compiled kernel instances. Each
// configuration lives in its own translation unit (built in parallel); the
// C-ABI layer dispatches to them by the planner's configuration index.
#pragma once

#include <hip/hip_runtime.h>

#include "ksplit_kernel.hpp"
#include "mx128_kernel.hpp"
#include "mx16_kernel.hpp"
#include "mx_kernel.hpp"
#include "mx_stream_kernel.hpp"
#include "skinny_kernel.hpp"
#include "stream_kernel.hpp"
#include "tile16_kernel.hpp"
#include "tile64_kernel.hpp"
#include "tile_kernel.hpp"

namespace tg {

struct Variant {
  bool b_col_major;
  bool out_bf16;
  bool debug;
};

template <int CFG>
hipError_t launch_tile(const TileArgs& a, int64_t grid, const Variant& v, hipStream_t stream);

template <int CFG>
hipError_t launch_skinny(const SkinnyArgs& a, int64_t grid, const Variant& v, hipStream_t stream);

template <int CFG>
hipError_t launch_mx(const MxArgs& a, int fmt, int64_t grid, const Variant& v, hipStream_t stream);

// Launch through hipLaunchKernel so the launch status comes back directly
// rather than through the thread's sticky last-error slot.
template <typename Args>
inline hipError_t launch_raw(const void* fn, dim3 grid, dim3 block, const Args& args,
                             hipStream_t stream) {
  void* argv[] = {const_cast<Args*>(&args)};
  return hipLaunchKernel(fn, grid, block, argv, 0, stream);
}

}  // namespace tg
