// host_abi.hpp -- the host-only half of the C ABI (include/tile_gemm.h):
// argument checks, planning and the tile map, with no HIP dependency.
//
// It is included by exactly one translation unit of the library
// (tile_gemm.hip, which adds the entry points that touch the device) and by
// the CPU test driver that builds these checks with the address and
// undefined-behaviour sanitizers. The checks follow the pages' contracts:
// argument errors are reported before anything is recorded and name the
// argument and axis ("Rust Compute Kernels", section "Shape contracts"); a
// written argument may not overlap another argument ("Rust Compute Kernels",
// section "Fusing invocations").
#pragma once

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "plan.hpp"
#include "tile_gemm.h"

namespace {

thread_local char g_detail[320];

tile_gemm_status_t fail(tile_gemm_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof g_detail, fmt, ap);
  va_end(ap);
  return s;
}

constexpr int64_t kMaxDim = (int64_t)1 << 31;

// B is row-major when its n stride is 1 and the k stride covers a row;
// otherwise column-major when its k stride is 1 and the n stride covers a
// column. (A vector B with both strides 1 is taken as row-major.)
bool b_is_row_major(const tile_gemm_strides_t* s, int64_t N) {
  return s->b_n == 1 && s->b_k >= N;
}
bool b_is_col_major(const tile_gemm_strides_t* s, int64_t K) {
  return s->b_k == 1 && s->b_n >= K;
}

// The instrumented kernel instances (write counter, colliding map) are needed
// only for those two flags; a forced configuration or grid runs the
// production instance, so forced runs time exactly what the planner launches.
bool instrumented(int flags) {
  return (flags & (TILE_GEMM_DEBUG_COUNT_WRITES | TILE_GEMM_DEBUG_COLLIDE)) != 0;
}

bool overlap(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) {
  return a0 < a1 && b0 < b1 && a0 < b1 && b0 < a1;
}

// Bytes from the first to one past the last element touched by `rows` rows of
// `extent` elements, `stride` elements apart: esz * ((rows - 1) * stride +
// extent). -1 when that overflows int64 (the caller then refuses the call).
int64_t span_bytes(int64_t rows, int64_t stride, int64_t extent, int64_t esz) {
  int64_t t, u, v;
  if (__builtin_mul_overflow(rows - 1, stride, &t) || __builtin_add_overflow(t, extent, &u) ||
      __builtin_mul_overflow(u, esz, &v))
    return -1;
  return v;
}

// n_out: C's width (N, or N/2 for SiLU(gate) * up); -1 means N.
tile_gemm_status_t check_args(const void* A, const void* B, const void* C, int64_t M, int64_t N,
                              int64_t K, const tile_gemm_strides_t* s, int dtype,
                              int64_t n_out = -1) {
  if (n_out < 0) n_out = N;
  g_detail[0] = '\0';
  if (dtype != TILE_GEMM_BF16_TO_F32 && dtype != TILE_GEMM_BF16_TO_BF16)
    return fail(TILE_GEMM_ERR_DTYPE, "dtype: unknown value %d", dtype);
  if (M < 0 || N < 0 || K < 0)
    return fail(TILE_GEMM_ERR_BAD_SHAPE, "shape: M=%lld N=%lld K=%lld, each must be >= 0",
                (long long)M, (long long)N, (long long)K);
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
    return fail(TILE_GEMM_ERR_BAD_SHAPE, "shape: M=%lld N=%lld K=%lld, each must be < 2^31",
                (long long)M, (long long)N, (long long)K);
  if (!s) return fail(TILE_GEMM_ERR_NULL_ARG, "strides: NULL");
  if (M == 0 || N == 0) return TILE_GEMM_OK;
  if (K > 0 && !A) return fail(TILE_GEMM_ERR_NULL_ARG, "A: NULL");
  if (K > 0 && !B) return fail(TILE_GEMM_ERR_NULL_ARG, "B: NULL");
  if (!C) return fail(TILE_GEMM_ERR_NULL_ARG, "C: NULL");

  // With K == 0 neither A nor B is read, so only C's layout matters.
  const bool brow = K == 0 || b_is_row_major(s, N);
  if (K > 0) {
    if (s->a_k != 1 || s->a_m < K)
      return fail(TILE_GEMM_ERR_BAD_STRIDE,
                  "A strides (a_m=%lld, a_k=%lld): need a_k == 1 and a_m >= K=%lld",
                  (long long)s->a_m, (long long)s->a_k, (long long)K);
    const bool bcol = !brow && b_is_col_major(s, K);
    if (!brow && !bcol)
      return fail(TILE_GEMM_ERR_BAD_STRIDE,
                  "B strides (b_k=%lld, b_n=%lld): need b_n == 1 and b_k >= N=%lld (row-major) "
                  "or b_k == 1 and b_n >= K=%lld (column-major)",
                  (long long)s->b_k, (long long)s->b_n, (long long)N, (long long)K);
  }
  if (s->c_n != 1 || s->c_m < n_out)
    return fail(TILE_GEMM_ERR_BAD_STRIDE,
                "C strides (c_m=%lld, c_n=%lld): need c_n == 1 and c_m >= %lld (C's width)",
                (long long)s->c_m, (long long)s->c_n, (long long)n_out);
  // Leading dimensions below 2^31 elements: every span below is then a small
  // multiple of 2^62 at most, and the checked arithmetic of span_bytes
  // refuses the rest instead of letting a product wrap.
  if (s->c_m >= kMaxDim)
    return fail(TILE_GEMM_ERR_BAD_STRIDE, "C: c_m=%lld, must be < 2^31", (long long)s->c_m);
  if (K > 0) {
    if (s->a_m >= kMaxDim)
      return fail(TILE_GEMM_ERR_BAD_STRIDE, "A: a_m=%lld, must be < 2^31", (long long)s->a_m);
    if ((brow ? s->b_k : s->b_n) >= kMaxDim)
      return fail(TILE_GEMM_ERR_BAD_STRIDE, "B: %s=%lld, must be < 2^31", brow ? "b_k" : "b_n",
                  (long long)(brow ? s->b_k : s->b_n));
  }

  const int64_t esz = (dtype == TILE_GEMM_BF16_TO_F32) ? 4 : 2;
  if ((uintptr_t)C % 16) return fail(TILE_GEMM_ERR_MISALIGNED, "C: base pointer not 16-byte aligned");
  if ((s->c_m * esz) % 16)
    return fail(TILE_GEMM_ERR_MISALIGNED, "C: c_m=%lld elements is not a multiple of 16 bytes",
                (long long)s->c_m);
  const int64_t c_span = span_bytes(M, s->c_m, n_out, esz);
  const uintptr_t c0 = (uintptr_t)C, c1 = c0 + (uintptr_t)c_span;
  if (c_span < 0 || c1 < c0)
    return fail(TILE_GEMM_ERR_BAD_SHAPE, "C: its byte range overflows the address space");
  if (K == 0) return TILE_GEMM_OK;
  if ((uintptr_t)A % 16) return fail(TILE_GEMM_ERR_MISALIGNED, "A: base pointer not 16-byte aligned");
  if ((uintptr_t)B % 16) return fail(TILE_GEMM_ERR_MISALIGNED, "B: base pointer not 16-byte aligned");
  if ((s->a_m * 2) % 16)
    return fail(TILE_GEMM_ERR_MISALIGNED, "A: a_m=%lld elements is not a multiple of 16 bytes",
                (long long)s->a_m);
  const int64_t ldb = brow ? s->b_k : s->b_n;
  if ((ldb * 2) % 16)
    return fail(TILE_GEMM_ERR_MISALIGNED, "B: %s=%lld elements is not a multiple of 16 bytes",
                brow ? "b_k" : "b_n", (long long)ldb);

  // Byte extents actually touched.
  const int64_t a_span = span_bytes(M, s->a_m, K, 2);
  const int64_t b_span = brow ? span_bytes(K, s->b_k, N, 2) : span_bytes(N, s->b_n, K, 2);
  // the kernels address each operand with 32-bit byte offsets
  if (a_span < 0 || a_span >= ((int64_t)1 << 32))
    return fail(TILE_GEMM_ERR_BAD_SHAPE, "A: spans %lld bytes, must be below 4 GiB", (long long)a_span);
  if (b_span < 0 || b_span >= ((int64_t)1 << 32))
    return fail(TILE_GEMM_ERR_BAD_SHAPE, "B: spans %lld bytes, must be below 4 GiB", (long long)b_span);

  const uintptr_t a0 = (uintptr_t)A, b0 = (uintptr_t)B;
  const uintptr_t a1 = a0 + (uintptr_t)a_span;
  const uintptr_t b1 = b0 + (uintptr_t)b_span;
  if (overlap(c0, c1, a0, a1)) return fail(TILE_GEMM_ERR_ALIAS, "C overlaps A (C is written)");
  if (overlap(c0, c1, b0, b1)) return fail(TILE_GEMM_ERR_ALIAS, "C overlaps B (C is written)");
  return TILE_GEMM_OK;
}

// Checks of the fused epilogue's arguments (C and its strides already checked).
tile_gemm_status_t check_epilogue(const void* C, int64_t M, int64_t N,
                                  const tile_gemm_strides_t* s, int dtype, const float* bias,
                                  int act) {
  if (act < TILE_GEMM_ACT_NONE || act > TILE_GEMM_ACT_SWIGLU)
    return fail(TILE_GEMM_ERR_EPILOGUE, "act: unknown activation %d", act);
  const bool glu = act == TILE_GEMM_ACT_SWIGLU;
  if (glu && N % 16)
    return fail(TILE_GEMM_ERR_BAD_SHAPE,
                "N=%lld: SiLU(gate) * up needs B's column count (gate + up) a multiple of 16",
                (long long)N);
  if (!bias || M == 0 || N == 0) return TILE_GEMM_OK;
  if ((uintptr_t)bias % 16) return fail(TILE_GEMM_ERR_MISALIGNED, "bias: pointer not 16-byte aligned");
  const int64_t esz = dtype == TILE_GEMM_BF16_TO_BF16 ? 2 : 4;
  const int64_t n_out = glu ? N / 2 : N;
  // (this check is also an entry point of its own, so the spans are formed
  // with overflow checks rather than trusting strides checked elsewhere)
  const int64_t c_span = span_bytes(M, s->c_m, n_out, esz), q_span = span_bytes(1, 0, N, 4);
  if (M < 0 || N < 0 || c_span < 0 || q_span < 0)
    return fail(TILE_GEMM_ERR_BAD_SHAPE, "C or bias: its byte range overflows");
  const uintptr_t c0 = (uintptr_t)C, c1 = c0 + (uintptr_t)c_span;
  const uintptr_t q0 = (uintptr_t)bias, q1 = q0 + (uintptr_t)q_span;
  if (overlap(c0, c1, q0, q1)) return fail(TILE_GEMM_ERR_ALIAS, "bias overlaps C (C is written)");
  return TILE_GEMM_OK;
}

void fill_plan(const tg::Plan& p, tile_gemm_plan_t* out) {
  out->variant = p.variant;
  out->config = p.config;
  out->bm = p.bm;
  out->bn = p.bn;
  out->bk = p.bk;
  out->threads = p.threads;
  out->lds_bytes = p.lds_bytes;
  out->tiles_m = p.map.tiles_m;
  out->tiles_n = p.map.tiles_n;
  out->group_m = p.map.group_m;
  out->xcds = p.map.xcds;
  out->k_split = p.k_split;
  out->grid = p.grid;
  out->tiles = p.tiles;
}


// Checks of tile_gemm_run_mx's arguments (see the header).
tile_gemm_status_t check_mx(const void* A, const void* B, const void* C, int64_t M, int64_t N,
                            int64_t K, const tile_gemm_strides_t* s, const void* sa,
                            const void* sb, int64_t ls, int fmt, int dtype, const float* bias,
                            int act) {
  g_detail[0] = '\0';
  if (dtype != TILE_GEMM_BF16_TO_F32 && dtype != TILE_GEMM_BF16_TO_BF16)
    return fail(TILE_GEMM_ERR_DTYPE, "dtype: unknown value %d", dtype);
  if (fmt != TILE_GEMM_MX_E4M3 && fmt != TILE_GEMM_MX_E2M1)
    return fail(TILE_GEMM_ERR_DTYPE, "fmt: unknown MX format %d", fmt);
  const bool fp4 = fmt == TILE_GEMM_MX_E2M1;
  const int kps = fp4 ? 2 * tg::kMxBK : tg::kMxBK;  // K elements per 64-byte slab
  if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
    return fail(TILE_GEMM_ERR_BAD_SHAPE, "shape: M=%lld N=%lld K=%lld, each must be in [0, 2^31)",
                (long long)M, (long long)N, (long long)K);
  if (K % kps)
    return fail(TILE_GEMM_ERR_BAD_SHAPE, "K=%lld: this MX format needs K a multiple of %d",
                (long long)K, kps);
  const int64_t kb = fp4 ? K / 2 : K;  // bytes of K in a row
  if (!s) return fail(TILE_GEMM_ERR_NULL_ARG, "strides: NULL");
  if (act < TILE_GEMM_ACT_NONE || act > TILE_GEMM_ACT_SILU)
    return fail(TILE_GEMM_ERR_EPILOGUE, "act: %d is not available for the MX product", act);
  if (M == 0 || N == 0) return TILE_GEMM_OK;
  if (!C) return fail(TILE_GEMM_ERR_NULL_ARG, "C: NULL");
  if (K > 0) {
    if (!A) return fail(TILE_GEMM_ERR_NULL_ARG, "A: NULL");
    if (!B) return fail(TILE_GEMM_ERR_NULL_ARG, "B: NULL");
    if (!sa) return fail(TILE_GEMM_ERR_NULL_ARG, "a_scale: NULL");
    if (!sb) return fail(TILE_GEMM_ERR_NULL_ARG, "b_scale: NULL");
    if (s->a_k != 1 || s->a_m < kb)
      return fail(TILE_GEMM_ERR_BAD_STRIDE,
                  "A strides (a_m=%lld, a_k=%lld): need a_k == 1, a_m >= %lld bytes",
                  (long long)s->a_m, (long long)s->a_k, (long long)kb);
    if (s->b_k != 1 || s->b_n < kb)
      return fail(TILE_GEMM_ERR_BAD_STRIDE,
                  "B strides (b_k=%lld, b_n=%lld): the MX product takes B as N x K, b_k == 1, "
                  "b_n >= %lld bytes",
                  (long long)s->b_k, (long long)s->b_n, (long long)kb);
    if (ls < K / 32 || ls % 4 || ls >= kMaxDim)
      return fail(TILE_GEMM_ERR_BAD_STRIDE,
                  "scale_stride=%lld: need a multiple of 4 bytes, >= K/32=%lld and < 2^31",
                  (long long)ls, (long long)(K / 32));
    if (s->a_m >= kMaxDim || s->b_n >= kMaxDim)
      return fail(TILE_GEMM_ERR_BAD_STRIDE, "A or B: a_m=%lld, b_n=%lld, each must be < 2^31",
                  (long long)s->a_m, (long long)s->b_n);
    // the kernels address scale rows (up to one tile past the edge) with
    // 32-bit byte offsets, formed as signed 32-bit products
    if ((M + 256) * ls >= kMaxDim || (N + 256) * ls >= kMaxDim)
      return fail(TILE_GEMM_ERR_BAD_SHAPE, "scales: rows x scale_stride must stay below 2 GiB");
  }
  if (s->c_n != 1 || s->c_m < N || s->c_m >= kMaxDim)
    return fail(TILE_GEMM_ERR_BAD_STRIDE,
                "C strides (c_m=%lld, c_n=%lld): need c_n == 1, N <= c_m < 2^31",
                (long long)s->c_m, (long long)s->c_n);
  const int64_t esz = dtype == TILE_GEMM_BF16_TO_F32 ? 4 : 2;
  if ((uintptr_t)C % 16) return fail(TILE_GEMM_ERR_MISALIGNED, "C: base pointer not 16-byte aligned");
  if ((s->c_m * esz) % 16)
    return fail(TILE_GEMM_ERR_MISALIGNED, "C: c_m=%lld elements is not a multiple of 16 bytes",
                (long long)s->c_m);
  const int64_t c_span = span_bytes(M, s->c_m, N, esz);
  const uintptr_t c0 = (uintptr_t)C, c1 = c0 + (uintptr_t)c_span;
  if (c_span < 0 || c1 < c0)
    return fail(TILE_GEMM_ERR_BAD_SHAPE, "C: its byte range overflows the address space");
  if (K > 0) {
    if ((uintptr_t)A % 16 || s->a_m % 16)
      return fail(TILE_GEMM_ERR_MISALIGNED, "A: base or a_m not a multiple of 16 bytes");
    if ((uintptr_t)B % 16 || s->b_n % 16)
      return fail(TILE_GEMM_ERR_MISALIGNED, "B: base or b_n not a multiple of 16 bytes");
    if ((uintptr_t)sa % 4 || (uintptr_t)sb % 4)
      return fail(TILE_GEMM_ERR_MISALIGNED, "scales: base pointers must be 4-byte aligned");
    const int64_t a_span = span_bytes(M, s->a_m, kb, 1), b_span = span_bytes(N, s->b_n, kb, 1);
    if (a_span < 0 || b_span < 0 || a_span >= ((int64_t)1 << 32) || b_span >= ((int64_t)1 << 32))
      return fail(TILE_GEMM_ERR_BAD_SHAPE, "A or B spans 4 GiB or more");
    const uintptr_t a0 = (uintptr_t)A, b0 = (uintptr_t)B, s0 = (uintptr_t)sa, t0 = (uintptr_t)sb;
    if (overlap(c0, c1, a0, a0 + a_span)) return fail(TILE_GEMM_ERR_ALIAS, "C overlaps A");
    if (overlap(c0, c1, b0, b0 + b_span)) return fail(TILE_GEMM_ERR_ALIAS, "C overlaps B");
    if (overlap(c0, c1, s0, s0 + (uintptr_t)(M * ls)))
      return fail(TILE_GEMM_ERR_ALIAS, "C overlaps a_scale");
    if (overlap(c0, c1, t0, t0 + (uintptr_t)(N * ls)))
      return fail(TILE_GEMM_ERR_ALIAS, "C overlaps b_scale");
  }
  return check_epilogue(C, M, N, s, dtype, bias, act);
}

}  // namespace

extern "C" {

const char* tile_gemm_status_str(tile_gemm_status_t s) {
  switch (s) {
    case TILE_GEMM_OK: return "ok";
    case TILE_GEMM_ERR_NULL_ARG: return "a required pointer is NULL";
    case TILE_GEMM_ERR_BAD_SHAPE: return "bad shape";
    case TILE_GEMM_ERR_BAD_STRIDE: return "unsupported strides";
    case TILE_GEMM_ERR_MISALIGNED: return "pointer or leading dimension not 16-byte aligned";
    case TILE_GEMM_ERR_ALIAS: return "output overlaps an input";
    case TILE_GEMM_ERR_DTYPE: return "unknown dtype";
    case TILE_GEMM_ERR_DEVICE: return "device unavailable, not gfx950, or not current";
    case TILE_GEMM_ERR_HIP: return "HIP runtime error";
    case TILE_GEMM_ERR_EPILOGUE: return "activation unknown or not available here";
  }
  return "unknown status";
}

const char* tile_gemm_last_error_detail(void) { return g_detail; }

tile_gemm_status_t tile_gemm_check_args(const void* A, const void* B, const void* C, int64_t M,
                                        int64_t N, int64_t K, const tile_gemm_strides_t* strides,
                                        tile_gemm_dtype_t dtype) {
  return check_args(A, B, C, M, N, K, strides, (int)dtype);
}

tile_gemm_status_t tile_gemm_check_epilogue(const void* C, int64_t M, int64_t N,
                                            const tile_gemm_strides_t* strides,
                                            tile_gemm_dtype_t dtype, const float* bias,
                                            tile_gemm_act_t act) {
  g_detail[0] = '\0';
  if (!strides) return fail(TILE_GEMM_ERR_NULL_ARG, "strides: NULL");
  return check_epilogue(C, M, N, strides, (int)dtype, bias, (int)act);
}

tile_gemm_status_t tile_gemm_check_mx(const void* A, const void* B, const void* C, int64_t M,
                                      int64_t N, int64_t K, const tile_gemm_strides_t* strides,
                                      const void* a_scale, const void* b_scale,
                                      int64_t scale_stride, tile_gemm_mx_format_t fmt,
                                      tile_gemm_dtype_t dtype, const float* bias,
                                      tile_gemm_act_t act) {
  return check_mx(A, B, C, M, N, K, strides, a_scale, b_scale, scale_stride, (int)fmt, (int)dtype,
                  bias, (int)act);
}

tile_gemm_status_t tile_gemm_plan_mx(int64_t M, int64_t N, int64_t K, tile_gemm_mx_format_t fmt,
                                     int cu_count, tile_gemm_plan_t* out) {
  g_detail[0] = '\0';
  if (!out) return fail(TILE_GEMM_ERR_NULL_ARG, "out: NULL");
  if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
    return fail(TILE_GEMM_ERR_BAD_SHAPE, "shape out of range");
  if (fmt != TILE_GEMM_MX_E4M3 && fmt != TILE_GEMM_MX_E2M1)
    return fail(TILE_GEMM_ERR_DTYPE, "fmt: unknown MX format %d", (int)fmt);
  if (cu_count <= 0) return fail(TILE_GEMM_ERR_DEVICE, "cu_count: %d", cu_count);
  fill_plan(tg::make_plan_mx(M, N, K, fmt == TILE_GEMM_MX_E2M1, cu_count), out);
  return TILE_GEMM_OK;
}

tile_gemm_status_t tile_gemm_plan(int64_t M, int64_t N, int64_t K, int b_col_major, int cu_count,
                                  tile_gemm_plan_t* out) {
  g_detail[0] = '\0';
  if (!out) return fail(TILE_GEMM_ERR_NULL_ARG, "out: NULL");
  if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
    return fail(TILE_GEMM_ERR_BAD_SHAPE, "shape out of range");
  if (cu_count <= 0) return fail(TILE_GEMM_ERR_DEVICE, "cu_count: %d", cu_count);
  fill_plan(tg::make_plan(M, N, K, b_col_major != 0, cu_count), out);
  return TILE_GEMM_OK;
}

tile_gemm_status_t tile_gemm_tile_of(const tile_gemm_plan_t* plan, int64_t M, int64_t N,
                                     int64_t wg, int64_t* m0, int64_t* n0, int64_t* rows,
                                     int64_t* cols) {
  g_detail[0] = '\0';
  if (!plan || !m0 || !n0 || !rows || !cols) return fail(TILE_GEMM_ERR_NULL_ARG, "NULL argument");
  if (wg < 0 || wg >= plan->tiles) return fail(TILE_GEMM_ERR_BAD_SHAPE, "tile index out of range");
  int64_t r0, c0;
  if (plan->variant == TILE_GEMM_VARIANT_TILE || plan->variant == TILE_GEMM_VARIANT_MX) {
    tg::TileMap mp{plan->tiles_m, plan->tiles_n, plan->group_m, plan->xcds};
    int32_t tm, tn;
    tg::tile_of(mp, (int32_t)wg, tm, tn);
    r0 = (int64_t)tm * plan->bm;
    c0 = (int64_t)tn * plan->bn;
    *rows = (r0 + plan->bm <= M) ? plan->bm : (M > r0 ? M - r0 : 0);
  } else if (plan->variant == TILE_GEMM_VARIANT_SKINNY) {
    r0 = 0;
    c0 = wg * plan->bn;
    *rows = M;
  } else {
    return fail(TILE_GEMM_ERR_BAD_SHAPE, "plan launches nothing");
  }
  *m0 = r0;
  *n0 = c0;
  *cols = (c0 + plan->bn <= N) ? plan->bn : (N > c0 ? N - c0 : 0);
  return TILE_GEMM_OK;
}

}  // extern "C"
