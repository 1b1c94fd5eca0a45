// tile_gemm.hip -- the C ABI (include/tile_gemm.h): the entry points that
// touch the device (create, run and its variants). Argument checks, planning
// and the tile map are host-only code in host_abi.hpp, included here.
//
// Conventions follow the pages:
//  * create is one-time preparation and run only records work on a stream
//    ("Rust Compute Kernels": prepare compiles or hits the cache once, record
//    only appends; "GPU speed, without leaving Rust's safety model", section
//    "Build once, choose how to execute");
//  * run allocates nothing, so it can be captured into a graph ("Why scoped
//    graph capture helps borrowing": capture is limited to non-allocating
//    operations);
//  * argument errors are reported before anything is recorded and name the
//    argument and axis ("Rust Compute Kernels", section "Shape contracts");
//  * a written argument may not overlap another argument ("Rust Compute
//    Kernels", section "Fusing invocations", which rejects exactly that).
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>

#include "launch.hpp"  // first: the HIP runtime headers plan.hpp relies on under hipcc
#include "host_abi.hpp"

struct tile_gemm_handle {
  int device;
  int cu_count;
  // TILE_GEMM_LOG=1 at create: the chosen plan is printed to stderr once per
  // shape (the first kLogShapes shapes; every call after that). A fixed table,
  // so run still allocates nothing.
  bool log;
  std::mutex log_mu;
  int n_logged;
  uint64_t logged[64];
};

namespace {

constexpr int kLogShapes = 64;

void log_plan(tile_gemm_handle* h, const char* kind, int64_t M, int64_t N, int64_t K, int layout,
              int dtype, int act, const tg::Plan& p) {
  if (!h->log) return;
  uint64_t key = 1469598103934665603ull;  // FNV-1a over the call's kind and shape
  for (const char* c = kind; *c; ++c) key = (key ^ (uint64_t)(unsigned char)*c) * 1099511628211ull;
  const int64_t parts[6] = {M, N, K, layout, dtype, act};
  for (int64_t v : parts)
    for (int b = 0; b < 8; ++b) key = (key ^ (uint64_t)((v >> (8 * b)) & 0xff)) * 1099511628211ull;
  std::lock_guard<std::mutex> lock(h->log_mu);
  for (int i = 0; i < h->n_logged; ++i)
    if (h->logged[i] == key) return;
  if (h->n_logged < kLogShapes) h->logged[h->n_logged++] = key;
  static const char* const kVariant[] = {"none", "tile", "skinny", "mx"};
  fprintf(stderr,
          "tile_gemm: %s M=%lld N=%lld K=%lld B=%s dtype=%d act=%d -> %s config %d, tile %dx%d, "
          "K step %d, %d threads, %lld tiles, grid %lld, k_split %d, group_m %d\n",
          kind, (long long)M, (long long)N, (long long)K, layout ? "column-major" : "row-major", dtype,
          act, kVariant[p.variant & 3], p.config, p.bm, p.bn, p.bk, p.threads, (long long)p.tiles,
          (long long)p.grid, p.k_split, p.map.group_m);
}

hipError_t dispatch_tile(int cfg, const tg::TileArgs& a, int64_t grid, const tg::Variant& v,
                         hipStream_t st) {
  switch (cfg) {
    case 0: return tg::launch_tile<0>(a, grid, v, st);
    case 1: return tg::launch_tile<1>(a, grid, v, st);
    case 2: return tg::launch_tile<2>(a, grid, v, st);
    case 3: return tg::launch_tile<3>(a, grid, v, st);
    case 4: return tg::launch_tile<4>(a, grid, v, st);
    case 5: return tg::launch_tile<5>(a, grid, v, st);
    case 6: return tg::launch_tile<6>(a, grid, v, st);
    case 7: return tg::launch_tile<7>(a, grid, v, st);
    case 8: return tg::launch_tile<8>(a, grid, v, st);
    case 9: return tg::launch_tile<9>(a, grid, v, st);
    case 10: return tg::launch_tile<10>(a, grid, v, st);
    case 11: return tg::launch_tile<11>(a, grid, v, st);
    case 12: return tg::launch_tile<12>(a, grid, v, st);
    case 13: return tg::launch_tile<13>(a, grid, v, st);
    case 14: return tg::launch_tile<14>(a, grid, v, st);
    case 15: return tg::launch_tile<15>(a, grid, v, st);
    case 16: return tg::launch_tile<16>(a, grid, v, st);
    case 17: return tg::launch_tile<17>(a, grid, v, st);
    case 18: return tg::launch_tile<18>(a, grid, v, st);
    case 19: return tg::launch_tile<19>(a, grid, v, st);
    case 20: return tg::launch_tile<20>(a, grid, v, st);
    case 21: return tg::launch_tile<21>(a, grid, v, st);
    case 22: return tg::launch_tile<22>(a, grid, v, st);
    case 23: return tg::launch_tile<23>(a, grid, v, st);
    case 24: return tg::launch_tile<24>(a, grid, v, st);
    case 25: return tg::launch_tile<25>(a, grid, v, st);
    case 26: return tg::launch_tile<26>(a, grid, v, st);
    case 27: return tg::launch_tile<27>(a, grid, v, st);
    case 28: return tg::launch_tile<28>(a, grid, v, st);
  }
  return hipErrorInvalidValue;
}
static_assert(tg::kNumTileConfigs == 29, "dispatch_tile covers every tile configuration");

hipError_t dispatch_skinny(int cfg, const tg::SkinnyArgs& a, int64_t grid, const tg::Variant& v,
                           hipStream_t st) {
  switch (cfg) {
    case 0: return tg::launch_skinny<0>(a, grid, v, st);
    case 1: return tg::launch_skinny<1>(a, grid, v, st);
    case 2: return tg::launch_skinny<2>(a, grid, v, st);
    case 3: return tg::launch_skinny<3>(a, grid, v, st);
    case 4: return tg::launch_skinny<4>(a, grid, v, st);
    case 5: return tg::launch_skinny<5>(a, grid, v, st);
  }
  return hipErrorInvalidValue;
}
static_assert(tg::kNumSkinnyConfigs == 6, "dispatch_skinny covers every skinny configuration");

hipError_t dispatch_mx(int cfg, const tg::MxArgs& a, int fmt, int64_t grid, const tg::Variant& v,
                       hipStream_t st) {
  switch (cfg) {
    case 0: return tg::launch_mx<0>(a, fmt, grid, v, st);
    case 1: return tg::launch_mx<1>(a, fmt, grid, v, st);
    case 2: return tg::launch_mx<2>(a, fmt, grid, v, st);
    case 3: return tg::launch_mx<3>(a, fmt, grid, v, st);
    case 4: return tg::launch_mx<4>(a, fmt, grid, v, st);
    case 5: return tg::launch_mx<5>(a, fmt, grid, v, st);
    case 6: return tg::launch_mx<6>(a, fmt, grid, v, st);
    case 7: return tg::launch_mx<7>(a, fmt, grid, v, st);
  }
  return hipErrorInvalidValue;
}
static_assert(tg::kNumMxConfigs == 8, "dispatch_mx covers every MX configuration");

tile_gemm_status_t run_mx_impl(tile_gemm_t h, const void* A, const void* B, void* C, int64_t M,
                               int64_t N, int64_t K, const tile_gemm_strides_t* s, const void* sa,
                               const void* sb, int64_t ls, int fmt, int dtype, const float* bias,
                               int act, void* stream, uint32_t* counts, int flags) {
  if (!h) return fail(TILE_GEMM_ERR_NULL_ARG, "handle: NULL");
  tile_gemm_status_t st = check_mx(A, B, C, M, N, K, s, sa, sb, ls, fmt, dtype, bias, act);
  if (st != TILE_GEMM_OK) return st;
  if (flags & ~(TILE_GEMM_DEBUG_COUNT_WRITES | TILE_GEMM_DEBUG_COLLIDE | 0x7f00ff00))
    return fail(TILE_GEMM_ERR_BAD_SHAPE, "flags: unknown bits 0x%x", flags);
  if (M == 0 || N == 0) return TILE_GEMM_OK;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != h->device)
    return fail(TILE_GEMM_ERR_DEVICE, "current device %d is not the handle's device %d", cur,
                h->device);
  if ((flags & TILE_GEMM_DEBUG_COUNT_WRITES) && !counts)
    return fail(TILE_GEMM_ERR_NULL_ARG, "counts: NULL with TILE_GEMM_DEBUG_COUNT_WRITES");
  tg::Plan p = tg::make_plan_mx(M, N, K, fmt == TILE_GEMM_MX_E2M1, h->cu_count);
  const int force = (flags >> 8) & 0xff;
  if (force) {
    if (force > tg::kNumMxConfigs)
      return fail(TILE_GEMM_ERR_BAD_SHAPE, "debug: no MX configuration %d", force - 1);
    if (tg::kMxConfigs[force - 1].mi == 16 && K % 128 != 0)
      return fail(TILE_GEMM_ERR_BAD_SHAPE, "debug: MX configuration %d needs K a multiple of 128",
                  force - 1);
    p = tg::plan_for_mx(force - 1, M, N, h->cu_count);
  }
  const int force_grid = (flags >> 24) & 0x7f;
  if (force_grid) p.grid = (force_grid == 0x7f || force_grid > p.tiles) ? p.tiles : force_grid;
  if ((flags & TILE_GEMM_DEBUG_COLLIDE) && p.tiles < 2)
    return fail(TILE_GEMM_ERR_BAD_SHAPE, "debug collide: needs >= 2 tiles");
  if (p.grid > 0x7fffffff) return fail(TILE_GEMM_ERR_BAD_SHAPE, "shape: too many workgroups");
  tg::MxArgs a{};
  a.A = static_cast<const uint8_t*>(A);
  a.B = static_cast<const uint8_t*>(B);
  a.sA = static_cast<const uint8_t*>(sa);
  a.sB = static_cast<const uint8_t*>(sb);
  a.C = C;
  a.M = (int32_t)M;
  a.N = (int32_t)N;
  a.K = (int32_t)K;
  a.lda = s->a_m;
  a.ldb = s->b_n;
  a.ldc = s->c_m;
  a.ls = (int32_t)ls;
  a.map = p.map;
  a.counts = counts;
  a.flags = flags;
  a.bias = bias;
  a.act = act;
  log_plan(h, fmt == TILE_GEMM_MX_E2M1 ? "run_mx e2m1" : "run_mx e4m3", M, N, K, 1, (int)dtype, act, p);
  const tg::Variant v{true, dtype == TILE_GEMM_BF16_TO_BF16, instrumented(flags)};
  const hipError_t e =
      dispatch_mx(p.config, a, fmt, p.grid, v, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(TILE_GEMM_ERR_HIP, "launch: %s", hipGetErrorString(e));
  return TILE_GEMM_OK;
}

tile_gemm_status_t run_impl(tile_gemm_t h, const void* A, const void* B, void* C, int64_t M,
                            int64_t N, int64_t K, const tile_gemm_strides_t* s,
                            tile_gemm_dtype_t dtype, void* stream, uint32_t* counts, int flags,
                            const float* bias = nullptr, int act = TILE_GEMM_ACT_NONE) {
  if (!h) return fail(TILE_GEMM_ERR_NULL_ARG, "handle: NULL");
  const bool glu = act == TILE_GEMM_ACT_SWIGLU;
  tile_gemm_status_t st = check_args(A, B, C, M, N, K, s, (int)dtype, glu ? N / 2 : N);
  if (st != TILE_GEMM_OK) return st;
  st = check_epilogue(C, M, N, s, (int)dtype, bias, act);
  if (st != TILE_GEMM_OK) return st;
  if (M == 0 || N == 0) return TILE_GEMM_OK;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != h->device)
    return fail(TILE_GEMM_ERR_DEVICE, "current device %d is not the handle's device %d", cur,
                h->device);
  if ((flags & TILE_GEMM_DEBUG_COUNT_WRITES) && !counts)
    return fail(TILE_GEMM_ERR_NULL_ARG, "counts: NULL with TILE_GEMM_DEBUG_COUNT_WRITES");

  const bool brow = K == 0 || b_is_row_major(s, N);
  tg::Plan p = tg::make_plan(M, N, K, !brow, h->cu_count);
  const int force_tile = (flags >> 8) & 0xff, force_skinny = (flags >> 16) & 0xff;
  if (force_tile && force_skinny)
    return fail(TILE_GEMM_ERR_BAD_SHAPE, "debug: force one configuration only");
  if (force_tile) {
    if (force_tile > tg::kNumTileConfigs)
      return fail(TILE_GEMM_ERR_BAD_SHAPE, "debug: no tile configuration %d", force_tile - 1);
    p = tg::plan_for(1, force_tile - 1, M, N, h->cu_count);
  } else if (force_skinny) {
    if (force_skinny > tg::kNumSkinnyConfigs)
      return fail(TILE_GEMM_ERR_BAD_SHAPE, "debug: no skinny configuration %d", force_skinny - 1);
    if (M > 16 * tg::kSkinnyConfigs[force_skinny - 1].mg)
      return fail(TILE_GEMM_ERR_BAD_SHAPE, "debug: M=%lld exceeds skinny configuration %d",
                  (long long)M, force_skinny - 1);
    p = tg::plan_for(2, force_skinny - 1, M, N, h->cu_count);
  }
  if (p.variant == 1 && tg::kTileConfigs[p.config].sb && (brow || K % 2))
    return fail(TILE_GEMM_ERR_BAD_SHAPE,
                "debug: tile configuration %d (stream kernel) takes a column-major B and an "
                "even K only",
                p.config);
  if (p.grid > 0x7fffffff)
    return fail(TILE_GEMM_ERR_BAD_SHAPE, "shape: %lld workgroups exceed the launch limit",
                (long long)p.grid);
  const int force_group = (flags >> 2) & 0x3f;
  if (force_group) {
    if (p.variant != 1)
      return fail(TILE_GEMM_ERR_BAD_SHAPE, "debug: a raster group applies to the tile kernel only");
    // any height >= 1 keeps tile_of a bijection (the last group may be short)
    p.map.group_m = force_group < p.map.tiles_m ? force_group : p.map.tiles_m;
  }
  const int force_grid = (flags >> 24) & 0x7f;
  if (force_grid) {
    if (p.variant != 1)
      return fail(TILE_GEMM_ERR_BAD_SHAPE, "debug: a forced grid applies to the tile kernel only");
    p.grid = (force_grid == 0x7f || force_grid > p.tiles) ? p.tiles : force_grid;
  }
  if ((flags & TILE_GEMM_DEBUG_COLLIDE) && (p.variant != 1 || p.tiles < 2))
    return fail(TILE_GEMM_ERR_BAD_SHAPE, "debug collide: needs the tile kernel and >= 2 tiles");

  log_plan(h, "run", M, N, K, !brow, (int)dtype, act, p);
  const tg::Variant v{!brow, dtype == TILE_GEMM_BF16_TO_BF16, instrumented(flags)};
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (p.variant == 1) {
    tg::TileArgs a{};
    a.A = static_cast<const uint16_t*>(A);
    a.B = static_cast<const uint16_t*>(B);
    a.C = C;
    a.M = (int32_t)M;
    a.N = (int32_t)N;
    a.K = (int32_t)K;
    a.lda = s->a_m;
    a.ldb = brow ? s->b_k : s->b_n;
    a.ldc = s->c_m;
    a.map = p.map;
    a.counts = counts;
    a.flags = flags;
    a.bias = bias;
    a.act = act;
    a.glu_half = glu ? (int32_t)(N / 2) : 0;
    e = dispatch_tile(p.config, a, p.grid, v, hs);
  } else {
    tg::SkinnyArgs a{};
    a.A = static_cast<const uint16_t*>(A);
    a.B = static_cast<const uint16_t*>(B);
    a.C = C;
    a.M = (int32_t)M;
    a.N = (int32_t)N;
    a.K = (int32_t)K;
    a.lda = s->a_m;
    a.ldb = brow ? s->b_k : s->b_n;
    a.ldc = s->c_m;
    a.counts = counts;
    a.flags = flags;
    a.bias = bias;
    a.act = act;
    a.glu_half = glu ? (int32_t)(N / 2) : 0;
    e = dispatch_skinny(p.config, a, p.grid, v, hs);
  }
  if (e != hipSuccess) return fail(TILE_GEMM_ERR_HIP, "launch: %s", hipGetErrorString(e));
  return TILE_GEMM_OK;
}

}  // namespace

extern "C" {

tile_gemm_status_t tile_gemm_create(tile_gemm_t* out, int device) {
  g_detail[0] = '\0';
  if (!out) return fail(TILE_GEMM_ERR_NULL_ARG, "out: NULL");
  *out = nullptr;
  int n = 0;
  const hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n <= 0)
    return fail(TILE_GEMM_ERR_DEVICE, "no HIP device visible (%s)", hipGetErrorString(e));
  if (device < 0 || device >= n)
    return fail(TILE_GEMM_ERR_DEVICE, "device %d out of range [0, %d)", device, n);
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess)
    return fail(TILE_GEMM_ERR_DEVICE, "cannot query device %d", device);
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(TILE_GEMM_ERR_DEVICE, "device %d is %s, not gfx950", device, prop.gcnArchName);
  tile_gemm_handle* hnd = new (std::nothrow) tile_gemm_handle{};
  if (!hnd) return fail(TILE_GEMM_ERR_HIP, "out of host memory");
  hnd->device = device;
  hnd->cu_count = prop.multiProcessorCount;
  const char* lg = getenv("TILE_GEMM_LOG");
  hnd->log = lg && lg[0] && strcmp(lg, "0") != 0;
  *out = hnd;
  return TILE_GEMM_OK;
}

tile_gemm_status_t tile_gemm_destroy(tile_gemm_t h) {
  delete h;
  return TILE_GEMM_OK;
}

tile_gemm_status_t tile_gemm_run(tile_gemm_t h, const void* A, const void* B, void* C, int64_t M,
                                 int64_t N, int64_t K, const tile_gemm_strides_t* strides,
                                 tile_gemm_dtype_t dtype, void* stream) {
  return run_impl(h, A, B, C, M, N, K, strides, dtype, stream, nullptr, 0);
}

tile_gemm_status_t tile_gemm_run_epilogue(tile_gemm_t h, const void* A, const void* B, void* C,
                                          int64_t M, int64_t N, int64_t K,
                                          const tile_gemm_strides_t* strides,
                                          tile_gemm_dtype_t dtype, const float* bias,
                                          tile_gemm_act_t act, void* stream) {
  return run_impl(h, A, B, C, M, N, K, strides, dtype, stream, nullptr, 0, bias, (int)act);
}

tile_gemm_status_t tile_gemm_run_debug(tile_gemm_t h, const void* A, const void* B, void* C,
                                       int64_t M, int64_t N, int64_t K,
                                       const tile_gemm_strides_t* strides, tile_gemm_dtype_t dtype,
                                       void* stream, uint32_t* counts, int flags,
                                       const float* bias, tile_gemm_act_t act) {
  if (flags & ~(TILE_GEMM_DEBUG_COUNT_WRITES | TILE_GEMM_DEBUG_COLLIDE | 0x7fffff00 | 0xfc))
    return fail(TILE_GEMM_ERR_BAD_SHAPE, "flags: unknown bits 0x%x", flags);
  return run_impl(h, A, B, C, M, N, K, strides, dtype, stream, counts, flags, bias, (int)act);
}

tile_gemm_status_t tile_gemm_run_mx(tile_gemm_t h, const void* A, const void* B, void* C,
                                    int64_t M, int64_t N, int64_t K,
                                    const tile_gemm_strides_t* strides, const void* a_scale,
                                    const void* b_scale, int64_t scale_stride,
                                    tile_gemm_mx_format_t fmt, tile_gemm_dtype_t dtype,
                                    const float* bias, tile_gemm_act_t act, void* stream) {
  return run_mx_impl(h, A, B, C, M, N, K, strides, a_scale, b_scale, scale_stride, (int)fmt,
                     (int)dtype, bias, (int)act, stream, nullptr, 0);
}

tile_gemm_status_t tile_gemm_run_mx_debug(tile_gemm_t h, const void* A, const void* B, void* C,
                                          int64_t M, int64_t N, int64_t K,
                                          const tile_gemm_strides_t* strides,
                                          const void* a_scale, const void* b_scale,
                                          int64_t scale_stride, tile_gemm_mx_format_t fmt,
                                          tile_gemm_dtype_t dtype, const float* bias,
                                          tile_gemm_act_t act, void* stream, uint32_t* counts,
                                          int flags) {
  return run_mx_impl(h, A, B, C, M, N, K, strides, a_scale, b_scale, scale_stride, (int)fmt,
                     (int)dtype, bias, (int)act, stream, counts, flags);
}

}  // extern "C"
