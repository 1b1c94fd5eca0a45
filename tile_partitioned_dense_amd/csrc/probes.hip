// probes.hip -- measurement probes for the roofline figures (not part of the
// GEMM library's ABI; built as its own small library, libtile_probes.so).
//
// Two ceilings the GEMM kernels are compared against on the same box, and the
// shader clock while a kernel runs:
//  * the rate at which the chip sustains bf16 MFMA instructions when nothing
//    else runs (no memory traffic, no LDS), with random or constant operands
//    and one or two waves per SIMD, for the 32x32x16 and 16x16x32 shapes,
//    and of the block-scaled FP8 (E4M3) forms 32x32x64 and 16x16x128;
//  * the rate at which HBM delivers a plain streaming read;
//  * the rate at which a compute unit's LDS serves 16-byte reads;
//  * the average shader clock over a window (a one-wave kernel beside the
//    measured work).
// Under sustained MFMA load the clock settles below the 2.4 GHz that the
// published peak assumes; the MFMA probe measures where it settles.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

namespace {

constexpr int kOps = 8;  // distinct operand registers per side

// Every wave loads kOps A and kOps B fragments (16 bytes per lane each) from
// `src` and then issues iters * 64 independent-chain MFMAs, rotating through
// the fragments so consecutive instructions see different data. 8 (or 16)
// accumulator chains keep every MFMA independent of the previous several.
template <int SHAPE>
__global__ __launch_bounds__(512) void mfma_probe(const u32x4* __restrict__ src, float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  bf16x8 a[kOps], b[kOps];
#pragma unroll
  for (int i = 0; i < kOps; ++i) {
    a[i] = __builtin_bit_cast(bf16x8, src[(wave * 2 * kOps + i) * 64 + lane]);
    b[i] = __builtin_bit_cast(bf16x8, src[(wave * 2 * kOps + kOps + i) * 64 + lane]);
  }
  float total = 0.0f;
  if constexpr (SHAPE == 0) {
    floatx16 acc[kOps];
#pragma unroll
    for (int i = 0; i < kOps; ++i) acc[i] = floatx16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < kOps; ++j)
#pragma unroll
        for (int i = 0; i < kOps; ++i)
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(i + j) % kOps], b[(5 * i + j) % kOps],
                                                            acc[i], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kOps; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) total += acc[i][e];
  } else {
    floatx4 acc[2 * kOps];
#pragma unroll
    for (int i = 0; i < 2 * kOps; ++i) acc[i] = floatx4{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < kOps; ++j)
#pragma unroll
        for (int i = 0; i < 2 * kOps; ++i)
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[(i + j) % kOps], b[(5 * i + j) % kOps],
                                                            acc[i], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2 * kOps; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) total += acc[i][e];
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = total;
}

// As mfma_probe for the block-scaled forms (SHAPE 0: 32x32x64, 1:
// 16x16x128) with E4M3 (FMT 0) or E2M1 (FMT 4: the first 16 bytes of each
// fragment) elements: 32-byte fragments (kF8Ops per side, so that fragments
// and accumulators fit the registers of two waves per SIMD without
// spilling), every scale byte 127 (a factor of 1).
constexpr int kF8Ops = 4;
template <int SHAPE, int FMT>
__global__ __launch_bounds__(512) void mfma_probe_f8(const u32x4* __restrict__ src, float* __restrict__ out,
                                                    int iters) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  i32x8 a[kF8Ops], b[kF8Ops];
#pragma unroll
  for (int i = 0; i < kF8Ops; ++i) {
    const u32x4 a0 = src[(wave * 4 * kF8Ops + 2 * i) * 64 + lane];
    const u32x4 a1 = src[(wave * 4 * kF8Ops + 2 * i + 1) * 64 + lane];
    const u32x4 b0 = src[(wave * 4 * kF8Ops + 2 * kF8Ops + 2 * i) * 64 + lane];
    const u32x4 b1 = src[(wave * 4 * kF8Ops + 2 * kF8Ops + 2 * i + 1) * 64 + lane];
    a[i] = i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    b[i] = i32x8{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  }
  constexpr int kScale = 127;
  float total = 0.0f;
  if constexpr (SHAPE == 0) {
    floatx16 acc[kOps];
#pragma unroll
    for (int i = 0; i < kOps; ++i) acc[i] = floatx16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < kOps; ++j)
#pragma unroll
        for (int i = 0; i < kOps; ++i)
          acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[(i + j) % kF8Ops], b[(3 * i + j) % kF8Ops],
                                                                   acc[i], FMT, FMT, 0, kScale, 0, kScale);
    }
#pragma unroll
    for (int i = 0; i < kOps; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) total += acc[i][e];
  } else {
    floatx4 acc[2 * kOps];
#pragma unroll
    for (int i = 0; i < 2 * kOps; ++i) acc[i] = floatx4{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < kOps; ++j)
#pragma unroll
        for (int i = 0; i < 2 * kOps; ++i)
          acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[(i + j) % kF8Ops], b[(3 * i + j) % kF8Ops],
                                                                    acc[i], FMT, FMT, 0, kScale, 0, kScale);
    }
#pragma unroll
    for (int i = 0; i < 2 * kOps; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) total += acc[i][e];
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = total;
}

// Streaming read of n16 16-byte units: workgroup g reads its own contiguous
// chunk (chunk = 1) or the whole grid strides through the buffer (chunk = 0),
// each lane 16 bytes per load, several loads in flight. The XOR of everything
// read is stored per thread so no load can be dropped.
__global__ __launch_bounds__(256) void read_probe(const u32x4* __restrict__ src, uint32_t* __restrict__ out, int64_t n16,
                           int chunk) {
  const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
  u32x4 x = {0u, 0u, 0u, 0u};
  if (chunk) {
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t lo = (int64_t)blockIdx.x * per;
    const int64_t hi = lo + per < n16 ? lo + per : n16;
    int64_t i = lo + threadIdx.x;
    for (; i + 3 * (int64_t)blockDim.x < hi; i += 4 * (int64_t)blockDim.x) {
      const u32x4 v0 = __builtin_nontemporal_load(src + i);
      const u32x4 v1 = __builtin_nontemporal_load(src + i + blockDim.x);
      const u32x4 v2 = __builtin_nontemporal_load(src + i + 2 * blockDim.x);
      const u32x4 v3 = __builtin_nontemporal_load(src + i + 3 * blockDim.x);
      x ^= v0 ^ v1 ^ v2 ^ v3;
    }
    for (; i < hi; i += blockDim.x) x ^= __builtin_nontemporal_load(src + i);
  } else {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * nthreads < n16; i += 4 * nthreads) {
      const u32x4 v0 = __builtin_nontemporal_load(src + i);
      const u32x4 v1 = __builtin_nontemporal_load(src + i + nthreads);
      const u32x4 v2 = __builtin_nontemporal_load(src + i + 2 * nthreads);
      const u32x4 v3 = __builtin_nontemporal_load(src + i + 3 * nthreads);
      x ^= v0 ^ v1 ^ v2 ^ v3;
    }
    for (; i < n16; i += nthreads) x ^= __builtin_nontemporal_load(src + i);
  }
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = x.x ^ x.y ^ x.z ^ x.w;
}

// One wave on one compute unit reads the shader-clock counter (s_memtime)
// and the constant-rate real-time counter (s_memrealtime) at its start, sleeps
// in short steps until `ticks` real-time ticks have passed, and reads both
// again: launched beside other work on a second stream it gives the average
// shader clock while that work runs. The wait is bounded by `ticks`.
__global__ __launch_bounds__(64) void clock_probe(unsigned long long* __restrict__ out,
                                                  long long ticks) {
  if (threadIdx.x != 0) return;
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  unsigned long long r1 = r0;
  while ((long long)(r1 - r0) < ticks) {
    __builtin_amdgcn_s_sleep(8);
    r1 = __builtin_amdgcn_s_memrealtime();
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  out[0] = c1 - c0;
  out[1] = r1 - r0;
}

}  // namespace

// LDS read rate: every wave of a 16-wave workgroup (one per compute unit)
// reads 16-byte chunks of a 64 KiB LDS buffer, eight reads in flight at a
// time, 64 consecutive chunks per wave-read (no bank conflicts); an empty asm
// statement takes the values, so no read is dropped or narrowed and no vector
// ALU work competes with the reads. `step` (in chunks, a kernel argument so
// the addresses stay in the loop) spaces a wave's eight reads.
__global__ __launch_bounds__(1024) void lds_probe(uint32_t* __restrict__ out, int iters, int step) {
  __shared__ u32x4 buf[4096];
  const int tid = threadIdx.x;
  for (int i = tid; i < 4096; i += blockDim.x)
    buf[i] = u32x4{(uint32_t)i, (uint32_t)(3 * i), (uint32_t)(5 * i), (uint32_t)(7 * i)};
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  int base = wave * 64 + lane;
  for (int it = 0; it < iters; ++it) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = buf[(base + u * step) & 4095];
    asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]));
    base += 8 * step;
  }
  out[blockIdx.x * blockDim.x + tid] = (uint32_t)base;
}

extern "C" {

// Launch the clock probe for `ticks` real-time ticks (at most 10^9; the
// real-time counter runs at hipDeviceAttributeWallClockRate kHz). out[0]
// receives the shader cycles elapsed, out[1] the real-time ticks.
int tg_probe_clock(unsigned long long* out, long long ticks, void* stream) {
  if (ticks <= 0 || ticks > 1000000000ll) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(clock_probe, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), out,
                     ticks);
  return (int)hipGetLastError();
}

// Launch the MFMA probe: `grid` workgroups of 4 * waves_per_simd waves (one
// workgroup per compute unit when grid = CU count), shape 0 = 32x32x16 bf16,
// 1 = 16x16x32 bf16, 2 = 32x32x64 scaled E4M3, 3 = 16x16x128 scaled E4M3,
// 4 = 32x32x64 scaled E2M1, 5 = 16x16x128 scaled E2M1.
// `src` holds at least grid * 4 * waves_per_simd * 16 KiB of operand bytes,
// `out` grid * 256 * waves_per_simd floats.
// Returns a hipError_t. FLOP per launch: waves * iters * 64 * 32768 for the
// bf16 shapes, four times that for the scaled ones (the 16x16 forms issue
// twice the instructions of half the size).
int tg_probe_mfma(const void* src, float* out, int grid, int waves_per_simd, int shape, int iters,
                  void* stream) {
  if (grid <= 0 || (waves_per_simd != 1 && waves_per_simd != 2) || shape < 0 || shape > 5 ||
      iters <= 0)
    return (int)hipErrorInvalidValue;
  const dim3 block(256 * waves_per_simd);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (shape == 0)
    hipLaunchKernelGGL(mfma_probe<0>, dim3(grid), block, 0, st, static_cast<const u32x4*>(src), out,
                       iters);
  else if (shape == 1)
    hipLaunchKernelGGL(mfma_probe<1>, dim3(grid), block, 0, st, static_cast<const u32x4*>(src), out,
                       iters);
  else if (shape == 2)
    hipLaunchKernelGGL((mfma_probe_f8<0, 0>), dim3(grid), block, 0, st, static_cast<const u32x4*>(src),
                       out, iters);
  else if (shape == 3)
    hipLaunchKernelGGL((mfma_probe_f8<1, 0>), dim3(grid), block, 0, st, static_cast<const u32x4*>(src),
                       out, iters);
  else if (shape == 4)
    hipLaunchKernelGGL((mfma_probe_f8<0, 4>), dim3(grid), block, 0, st, static_cast<const u32x4*>(src),
                       out, iters);
  else
    hipLaunchKernelGGL((mfma_probe_f8<1, 4>), dim3(grid), block, 0, st, static_cast<const u32x4*>(src),
                       out, iters);
  return (int)hipGetLastError();
}

// Launch the LDS probe: `grid` workgroups of 16 waves, each wave 8 * iters
// reads of 1 KiB; `out` holds grid * 1024 uint32. Returns a hipError_t.
int tg_probe_lds(uint32_t* out, int grid, int iters, int step, void* stream) {
  if (grid <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(lds_probe, dim3(grid), dim3(1024), 0, static_cast<hipStream_t>(stream), out, iters,
                     step);
  return (int)hipGetLastError();
}

// Launch the read probe over `bytes` (a multiple of 16) of `src`; `out` holds
// grid * 256 uint32. chunk: 1 = one contiguous chunk per workgroup, 0 =
// grid-strided. Returns a hipError_t.
int tg_probe_read(const void* src, uint32_t* out, int64_t bytes, int grid, int chunk,
                  void* stream) {
  if (grid <= 0 || bytes <= 0 || bytes % 16) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_probe, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), out, bytes / 16, chunk);
  return (int)hipGetLastError();
}

}  // extern "C"
