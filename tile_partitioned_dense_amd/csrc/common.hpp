// common.hpp -- vector types, bf16 helpers and MFMA wrappers for gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Fused-epilogue activations (mirror TILE_GEMM_ACT_* in tile_gemm.h).
constexpr int kActNone = 0, kActRelu = 1, kActSigmoid = 2, kActTanh = 3, kActSilu = 4,
              kActSwiglu = 5;

// e^x as 2^(x log2 e) on the hardware exponential (v_exp_f32, about 1 ulp):
// rounding x log2 e adds a relative error of about 2^-24 |x| to the result,
// the size of the rounding already present in an fp32 x.
__device__ __forceinline__ float exp_hw(float x) {
  return __builtin_amdgcn_exp2f(x * 1.44269504088896341f);
}

// 1 / (1 + e^-x) with the hardware reciprocal (about 1 ulp); saturates to
// exactly 0 and 1 where e^-x overflows or underflows.
__device__ __forceinline__ float sigmoid_hw(float x) {
  return __builtin_amdgcn_rcpf(1.0f + exp_hw(-x));
}

// tanh x. For |x| >= 1/2, 1 - 2 / (e^(2|x|) + 1) with the sign of x: the
// hardware exponential and reciprocal keep the absolute error near 1e-7,
// small against |tanh x| >= 0.46. Below 1/2 that difference would cancel, so
// the odd Taylor series of tanh (coefficients 2^(2n) (2^(2n) - 1) B_2n / (2n)!
// from the Bernoulli numbers: 1, -1/3, 2/15, -17/315, 62/2835,
// -1382/155925, 21844/6081075) through x^13 takes over; its truncation error
// there is below 1e-7 relative. Both are evaluated and one selected, so
// lanes on either side of 1/2 do not diverge.
__device__ __forceinline__ float tanh_hw(float x) {
  const float a = fabsf(x);
  const float z = a * a;
  float p = 21844.0f / 6081075.0f;
  p = p * z - 1382.0f / 155925.0f;
  p = p * z + 62.0f / 2835.0f;
  p = p * z - 17.0f / 315.0f;
  p = p * z + 2.0f / 15.0f;
  p = p * z - 1.0f / 3.0f;
  p = p * z + 1.0f;
  const float small = a * p;
  const float large = 1.0f - 2.0f * __builtin_amdgcn_rcpf(exp_hw(2.0f * a) + 1.0f);
  return copysignf(a < 0.5f ? small : large, x);
}

// act(x) in fp32 for a compile-time activation.
template <int ACT>
__device__ __forceinline__ float act_fn(float x) {
  if constexpr (ACT == kActRelu) return fmaxf(x, 0.0f);
  else if constexpr (ACT == kActSigmoid) return sigmoid_hw(x);
  else if constexpr (ACT == kActTanh) return tanh_hw(x);
  else if constexpr (ACT == kActSilu) return x * sigmoid_hw(x);
  else return x;
}

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

// Destination and epilogue of store_staged_fused.
struct EpiOut {
  void* C;
  int64_t ldc;
  int32_t M, N;
  const float* bias;
  int32_t act;
  uint32_t* counts;  // debug instrumentation only
  int32_t flags;
};

__device__ __forceinline__ floatx4 lds_load_f4(uint32_t addr) {
  return *(const __attribute__((address_space(3))) floatx4*)(uintptr_t)addr;
}
__device__ __forceinline__ void lds_store_f4(uint32_t addr, const floatx4& v) {
  *(__attribute__((address_space(3))) floatx4*)(uintptr_t)addr = v;
}

// The row loop of store_staged_fused for one activation (the activation is
// a template argument, so the loop carries no per-element dispatch).
template <bool OUT_BF16, bool DEBUG, int ACT>
__device__ __forceinline__ void store_staged_rows(uint32_t src, int pitch, int rows, int grow0,
                                                  int r0, int rstep, int ch, int col, bool full,
                                                  const float (&b)[OUT_BF16 ? 8 : 4],
                                                  const EpiOut& o) {
  constexpr int EPC = OUT_BF16 ? 8 : 4;
  constexpr int ESZ = OUT_BF16 ? 2 : 4;
  const int rend = rows < o.M - grow0 ? rows : o.M - grow0;
#pragma unroll 2
  for (int r = r0; r < rend; r += rstep) {
    float v[EPC];
#pragma unroll
    for (int h = 0; h < EPC / 4; ++h) {
      const floatx4 x = lds_load_f4(src + (uint32_t)(r * pitch + (ch * EPC + 4 * h) * 4));
      v[4 * h] = x[0]; v[4 * h + 1] = x[1]; v[4 * h + 2] = x[2]; v[4 * h + 3] = x[3];
    }
    if (o.bias) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) v[e] += b[e];
    }
#pragma unroll
    for (int e = 0; e < EPC; ++e) v[e] = act_fn<ACT>(v[e]);
    const int row = grow0 + r;
    char* cb = static_cast<char*>(o.C) + ((int64_t)row * o.ldc + col) * ESZ;
    if (full) {
      if constexpr (OUT_BF16) {
        *reinterpret_cast<uint4*>(cb) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                   pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
      } else {
        *reinterpret_cast<float4*>(cb) = make_float4(v[0], v[1], v[2], v[3]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        if (col + e < o.N) {
          if constexpr (OUT_BF16) {
            reinterpret_cast<uint16_t*>(cb)[e] = f32_to_bf16(v[e]);
          } else {
            reinterpret_cast<float*>(cb)[e] = v[e];
          }
        }
      }
    }
    if constexpr (DEBUG) {
      if (o.flags & kDbgCount)
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          if (col + e < o.N) atomicAdd(o.counts + (int64_t)row * o.N + col + e, 1u);
    }
  }
}

// Fused-epilogue store of an fp32 block staged row-major in LDS: `rows` x
// `cols` values at LDS byte address `src` (row pitch `pitch` bytes, both
// multiples of 16) belong at C[grow0 + r][gcol0 + c]. The block is cut into
// 16-byte output chunks (4 fp32 or 8 bf16 columns; `cols` is a multiple of 8
// and at most 8 * nthr) and thread `tid` of `nthr` keeps one chunk column
// for every row it visits, so it loads its bias once. Each element is formed
// as act(x + bias) in fp32, rounded to bf16 (nearest even) for a bf16 output
// and written once; rows and columns past M and N are masked. The row loop
// stays rolled (unrolled twice to overlap its LDS reads), so the activation
// code is emitted a fixed number of times however large the block.
template <bool OUT_BF16, bool DEBUG>
__device__ __forceinline__ void store_staged_fused(uint32_t src, int pitch, int rows, int cols,
                                                   int grow0, int gcol0, int tid, int nthr,
                                                   const EpiOut& o) {
  constexpr int EPC = OUT_BF16 ? 8 : 4;  // elements per 16-byte output chunk
  const int cho = cols / EPC;             // chunks per row
  const int rstep = nthr / cho;           // rows one pass of the threads covers
  if (tid >= rstep * cho) return;         // threads past a whole number of rows idle
  const int ch = tid % cho;
  const int col = gcol0 + ch * EPC;
  if (col >= o.N) return;
  const bool full = col + EPC <= o.N;
  float b[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) b[e] = 0.0f;
  if (o.bias) {
    if (full) {
#pragma unroll
      for (int h = 0; h < EPC / 4; ++h) {
        const float4 x = *reinterpret_cast<const float4*>(o.bias + col + 4 * h);
        b[4 * h] = x.x; b[4 * h + 1] = x.y; b[4 * h + 2] = x.z; b[4 * h + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e)
        if (col + e < o.N) b[e] = o.bias[col + e];
    }
  }
  switch (o.act) {
    case kActRelu:
      store_staged_rows<OUT_BF16, DEBUG, kActRelu>(src, pitch, rows, grow0, tid / cho, rstep, ch, col, full, b, o);
      break;
    case kActSigmoid:
      store_staged_rows<OUT_BF16, DEBUG, kActSigmoid>(src, pitch, rows, grow0, tid / cho, rstep, ch, col, full, b, o);
      break;
    case kActTanh:
      store_staged_rows<OUT_BF16, DEBUG, kActTanh>(src, pitch, rows, grow0, tid / cho, rstep, ch, col, full, b, o);
      break;
    case kActSilu:
      store_staged_rows<OUT_BF16, DEBUG, kActSilu>(src, pitch, rows, grow0, tid / cho, rstep, ch, col, full, b, o);
      break;
    default:
      store_staged_rows<OUT_BF16, DEBUG, kActNone>(src, pitch, rows, grow0, tid / cho, rstep, ch, col, full, b, o);
  }
}

// SiLU(gate) * up store of an fp32 gate+up block staged in LDS: block row r
// (0 <= r < rows) holds `cols` gate values followed by the `cols` matching up
// values, at LDS byte address src + r * pitch. Block row r is output row
// grow0 + (r / rgroup) * rgap + r % rgroup (several waves' strips side by
// side); block column c < cols is output column gcol0 + c of an output o.N
// (= half the product's columns) wide. The gate's bias is bias[j], the up
// value's bias[half + j]. Threads split the work as in store_staged_fused.
template <bool OUT_BF16, bool DEBUG>
__device__ __forceinline__ void store_staged_glu(uint32_t src, int pitch, int rows, int cols,
                                                 int rgroup, int rgap, int grow0, int gcol0,
                                                 int tid, int nthr, const EpiOut& o) {
  constexpr int EPC = OUT_BF16 ? 8 : 4;
  constexpr int ESZ = OUT_BF16 ? 2 : 4;
  const int cho = cols / EPC;
  const int rstep = nthr / cho;
  if (tid >= rstep * cho) return;
  const int ch = tid % cho;
  const int col = gcol0 + ch * EPC;
  if (col >= o.N) return;
  const bool full = col + EPC <= o.N;
  float bg[EPC], bu[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
    bg[e] = 0.0f;
    bu[e] = 0.0f;
  }
  if (o.bias) {
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      if (full || col + e < o.N) {
        bg[e] = o.bias[col + e];
        bu[e] = o.bias[o.N + col + e];
      }
    }
  }
#pragma unroll 2
  for (int r = tid / cho; r < rows; r += rstep) {
    const int row = grow0 + (r / rgroup) * rgap + (r - (r / rgroup) * rgroup);
    if (row >= o.M) continue;
    float g[EPC], u[EPC];
#pragma unroll
    for (int h = 0; h < EPC / 4; ++h) {
      const uint32_t a = src + (uint32_t)(r * pitch + (ch * EPC + 4 * h) * 4);
      const floatx4 x = lds_load_f4(a);
      const floatx4 y = lds_load_f4(a + (uint32_t)(cols * 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        g[4 * h + e] = x[e];
        u[4 * h + e] = y[e];
      }
    }
    float v[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const float gv = g[e] + bg[e], uv = u[e] + bu[e];
      v[e] = gv * sigmoid_hw(gv) * uv;
    }
    char* cb = static_cast<char*>(o.C) + ((int64_t)row * o.ldc + col) * ESZ;
    if (full) {
      if constexpr (OUT_BF16) {
        *reinterpret_cast<uint4*>(cb) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                   pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
      } else {
        *reinterpret_cast<float4*>(cb) = make_float4(v[0], v[1], v[2], v[3]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        if (col + e < o.N) {
          if constexpr (OUT_BF16) {
            reinterpret_cast<uint16_t*>(cb)[e] = f32_to_bf16(v[e]);
          } else {
            reinterpret_cast<float*>(cb)[e] = v[e];
          }
        }
      }
    }
    if constexpr (DEBUG) {
      if (o.flags & kDbgCount)
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          if (col + e < o.N) atomicAdd(o.counts + (int64_t)row * o.N + col + e, 1u);
    }
  }
}

}  // namespace tg
