// common.hpp -- vector types, bf16 helpers and MFMA wrappers for gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Debug flags (mirror TILE_GEMM_DEBUG_* in tile_gemm.h).
constexpr int kDbgCount = 1;
constexpr int kDbgCollide = 2;

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest, ties to even: gfx950 converts in hardware
// (v_cvt_pk_bf16_f32, two values per instruction, NaN -> quiet NaN). The
// packed form puts `lo` in bits 0-15 and `hi` in bits 16-31.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// 32x32x16 bf16 MFMA, fp32 accumulate. Lane l supplies row (l % 32) of the
// A block and column (l % 32) of the B block, each as 8 consecutive k values
// of k group (l / 32); lane l receives column (l % 32), rows
// 8*(v/4) + 4*(l/32) + (v%4) for accumulator element v.
__device__ __forceinline__ floatx16 mfma32(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16 MFMA: lane l supplies row / column (l % 16), k group (l / 16)
// of 8 values; receives column (l % 16), rows 4*(l/16) + v.
__device__ __forceinline__ floatx4 mfma16(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Eight consecutive bf16 of one row, zero beyond `len` valid elements. The
// vector path is taken only when all eight are in range (16-byte aligned by
// the argument checks); the tail is read element by element so no access
// leaves the row's valid extent.
__device__ __forceinline__ uint4 load8_masked(const uint16_t* row, int c, int len) {
  if (c + 8 <= len) return *reinterpret_cast<const uint4*>(row + c);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t v = (c + e < len) ? (uint32_t)row[c + e] : 0u;
    w[e >> 1] |= v << (16 * (e & 1));
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_nt __attribute__((ext_vector_type(2)));

// Streaming (non-temporal) loads for data read exactly once: the hardware
// keeps them from displacing reused lines in the caches.
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load8_stream(const void* p) {
  const u32x2_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_nt*>(p));
  return make_uint2(v.x, v.y);
}

// Pack the low (hi_half = false) or high halves of two dwords: the result
// holds x's half in bits 0-15 and y's half in bits 16-31.
__device__ __forceinline__ uint32_t pack_halves(uint32_t x, uint32_t y, bool hi_half) {
  return hi_half ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
}

}  // namespace tg
