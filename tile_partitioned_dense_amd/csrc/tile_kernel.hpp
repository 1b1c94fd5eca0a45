// tile_kernel.hpp -- the LDS-staged bf16 MFMA tile kernel for gfx950.
//
// Every BM x BN tile of C has exactly one owning workgroup (found with
// tile_of), its only writer; a workgroup owns one tile, or several taken one
// after the other when the planner launches fewer workgroups than tiles.
// Four or eight waves (one or two per SIMD) split the tile into
// WM x WN wave tiles. The workgroup walks K in 32-wide slabs in ascending
// order through a ring of NST LDS buffers:
//
//   global --(buffer load straight into LDS, no registers)--> LDS stage
//   LDS stage --(ds_read)--> MFMA operands --> fp32 accumulators
//
// and stores its tile once at the end. A and B are only read, so slabs are
// fetched up to NST - 1 ahead; C is never read.
//
// Pipeline (per wave, slab s, two 16-k steps kk = 0, 1):
//   MFMAs(s, 0)  while reading the operands of (s, 1) and issuing the second
//                half of this wave's loads of slab s + NST - 2
//   wait for this wave's loads of slab s + 1, barrier (every wave's loads of
//   slab s + 1 have landed, and every wave is done with slab s - 1)
//   MFMAs(s, 1)  while reading the operands of (s + 1, 0) and issuing the
//                first half of the loads of slab s + NST - 1 into the stage
//                slab s - 1 just freed
// Splitting each slab's loads over two steps keeps the texture unit's queue
// from filling (a wave that finds it full stalls, MFMAs included). The
// barrier is a bare s_barrier with explicit vmcnt waits: a full fence would
// also wait for the loads that are meant to stay in flight.
//
// Accumulators hold each 32 x 32 block of C transposed (see mma), so a lane
// owns four consecutive columns of one row. The epilogue stages each wave's
// results through the then idle ring and writes C as 16-byte row chunks.
//
// LDS layouts (all reads conflict-free on 64 banks):
//  * A, and B when column-major (both K-contiguous): a slab row is 32 bf16 =
//    64 bytes = four 16-byte chunks; chunk c of row r sits at position
//    c ^ ((r >> 2) & 3), so the 16 rows one MFMA read touches land in 16
//    distinct 16-byte bank groups.
//  * B row-major (N-contiguous): a slab is 32 k rows of BN bf16. MFMA wants 8
//    consecutive k per lane; ds_read_b64_tr_b16 delivers them: within each
//    group of 16 lanes, lane 4j + q names row j, columns 4q..4q+3 of a 4 x 16
//    block and receives column (lane % 16), rows 0..3. When the row pitch is a
//    multiple of 256 bytes, 64-byte block b of row k sits at b ^ (k & 3) so
//    the four rows one group reads hit different banks; other pitches already
//    stagger them.
//
// Bounds: each slab's buffer resources start at the slab and end at the last
// valid element of the operand, so rows (or, for a row-major B, columns) past
// the edge read as zero and no load can leave the operand. Values read for
// rows >= M or columns >= N only reach accumulators that are never stored. A
// K tail (K % 32 != 0) must be exact zeros in both operands; that one slab is
// fetched through registers with element masks and written to LDS with
// ds_write. The range check zeroes whole dwords: a dword that straddles the
// end of a resource reads as zero, including its valid half. Only the
// operand's very last value can sit in such a dword; for A and a column-major
// B it lies in the K tail whenever K is odd, and for a row-major B with an
// odd N the last slab (row K - 1) is sent through the register path as well.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "plan.hpp"

namespace tg {

struct TileArgs {
  const uint16_t* A;
  const uint16_t* B;
  void* C;
  int32_t M, N, K;
  int64_t lda;  // A: elements between rows
  int64_t ldb;  // row-major B: between k rows; column-major B: between n columns
  int64_t ldc;  // C: elements between rows
  TileMap map;
  uint32_t* counts;  // debug instrumentation only
  int32_t flags;     // debug instrumentation only
  const float* bias;  // fused epilogue: N fp32 values or NULL
  int32_t act;        // fused epilogue: kAct*
  int32_t glu_half;   // SiLU(gate) * up: N / 2 (the gate's width), else 0
};

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

constexpr int kTileBK = 32;  // K per slab

// Raw buffer resource over [base, base + bytes): loads beyond it return zero
// and touch no memory.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t n = bytes <= 0 ? 0u : (bytes > 0xffffffffll ? 0xffffffffu : (uint32_t)bytes);
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int32_t)((a >> 32) & 0xffffu));
  r.z = __builtin_amdgcn_readfirstlane((int32_t)n);
  r.w = 0x00020000;
  return r;
}

// 16 bytes per lane from rsrc + voff + soff straight into LDS at lds + 16 *
// lane (one contiguous KiB per wave). Tracked by vmcnt only. gfx9 LDS
// instructions do not read M0, and nothing else in these kernels sets it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ i32x4 uniform_rsrc(const i32x4& r) {
  i32x4 u;
  u.x = __builtin_amdgcn_readfirstlane(r.x);
  u.y = __builtin_amdgcn_readfirstlane(r.y);
  u.z = __builtin_amdgcn_readfirstlane(r.z);
  u.w = __builtin_amdgcn_readfirstlane(r.w);
  return u;
}
__device__ __forceinline__ void dma16(uint32_t lds, const i32x4& rsrc_in, uint32_t voff,
                                      uint32_t soff) {
  const i32x4 rsrc = uniform_rsrc(rsrc_in);
  lds = __builtin_amdgcn_readfirstlane(lds);
  soff = __builtin_amdgcn_readfirstlane(soff);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory", "m0");
}
// 4 bytes per lane from rsrc + voff + soff straight into LDS at lds + 4 *
// lane (256 contiguous bytes per wave). Tracked by vmcnt only.
__device__ __forceinline__ void dma4(uint32_t lds, const i32x4& rsrc_in, uint32_t voff,
                                     uint32_t soff) {
  const i32x4 rsrc = uniform_rsrc(rsrc_in);
  lds = __builtin_amdgcn_readfirstlane(lds);
  soff = __builtin_amdgcn_readfirstlane(soff);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dword %1, %2, %3 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// As dma16, with the LDS address formed as an SGPR base plus a constant.
// The addition happens outside the asm: the asm itself must not touch SCC,
// which the compiler may hold live across it (a loop condition, a carry).
template <uint32_t OFF>
__device__ __forceinline__ void dma16_off(uint32_t lds_base, const i32x4& rsrc, uint32_t voff) {
  dma16(lds_base + OFF, rsrc, voff, 0u);
}

// Move a buffer resource `step` bytes forward (base up, extent down, never
// below zero, so a resource moved past its end only yields out-of-range
// loads). Exact while the extent never needed clamping (operands < 4 GiB).
__device__ __forceinline__ void advance_rsrc(i32x4& r, uint32_t step) {
  uint64_t base = ((uint64_t)((uint32_t)r.y & 0xffffu) << 32) | (uint32_t)r.x;
  base += step;
  r.x = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)base);
  r.y = __builtin_amdgcn_readfirstlane((int32_t)((base >> 32) & 0xffffu));
  const uint32_t left = (uint32_t)r.z;
  r.z = __builtin_amdgcn_readfirstlane((int32_t)(left > step ? left - step : 0u));
}

// Compile-time loop: f(integral_constant<int, I>) for I in [I0, N).
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// s_waitcnt with only the vector-memory counter constrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int swzA(int r) { return (r >> 2) & 3; }

// 16-byte LDS read at a byte address.
__device__ __forceinline__ bf16x8 lds_read16(uint32_t addr) {
  return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)addr;
}

// One 32 x 32 x 16 step of a C block held transposed: the B fragment goes in
// as the MFMA's row operand and the A fragment as its column operand, so the
// MFMA computes the block of C^T. Lane l then holds C row (l % 32), columns
// 8 q + 4 (l / 32) + r in accumulator element 4 q + r: four consecutive
// columns per q, which the epilogue stores as one vector. Every output element
// is still the sum over the same 16 products.
__device__ __forceinline__ floatx16 mma(const bf16x8& a_frag, const bf16x8& b_frag, const floatx16& acc) {
  return mfma32(b_frag, a_frag, acc);
}

template <int BM, int BN, int WM, int WN, int NST, bool BCOL, bool OUT_BF16, bool DEBUG>
__global__ __launch_bounds__(WM * WN * 64, 1) void tile_gemm_kernel(TileArgs p) {
  constexpr int kStages = NST;  // LDS ring depth
  static_assert(NST >= 3 && NST <= 6, "ring depth");
  constexpr int NW = WM * WN;
  constexpr int NT = NW * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(NW == 4 || NW == 8, "one or two waves per SIMD");
  constexpr int BK = kTileBK;
  constexpr int A_BYTES = BM * BK * 2;  // per stage
  constexpr int B_BYTES = BN * BK * 2;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_DMA = A_BYTES / 1024;  // one KiB per wave instruction
  constexpr int B_DMA = B_BYTES / 1024;
  static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "slabs are whole KiB");
  static_assert(A_DMA % NW == 0, "A slab splits evenly over the waves");
  constexpr int A_PER = A_DMA / NW;
  constexpr int B_MAX = (B_DMA + NW - 1) / NW;  // B instructions of waves < B_DMA % NW
  constexpr int B_MIN = B_DMA / NW;
  constexpr int PITCH = BN * 2;  // row-major B: bytes per k row
  constexpr bool SWB = !BCOL && (PITCH % 256 == 0);
  constexpr int CPR = BN / 8;  // row-major B: 16-byte chunks per k row

  __shared__ __attribute__((aligned(1024))) uint4 smem[kStages * STAGE / 16];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave - (wave / WN) * WN;

  // Tiles wg = blockIdx.x, blockIdx.x + gridDim.x, ...: one per workgroup
  // when the grid covers every tile, several (always whole, each with its own
  // K loop and store) when the planner launches fewer workgroups than tiles.
  const int n_tiles = p.map.tiles_m * p.map.tiles_n;
  for (int wg_it = blockIdx.x; wg_it < n_tiles; wg_it += gridDim.x) {
    int wg = wg_it;
    if constexpr (DEBUG) {
      if ((p.flags & kDbgCollide) && wg == 1) wg = 0;  // negative control only
    }
    int32_t tm, tn;
    tile_of(p.map, wg, tm, tn);
    const int M = p.M, N = p.N, K = p.K;
    const int64_t lda = p.lda, ldb = p.ldb;
    // With SiLU(gate) * up the tile's first BN/2 columns are gate columns
    // n0 .. and its last BN/2 the up columns glu + n0 ..: B column n0 + c for
    // c < BN/2, glu - BN/2 + n0 + c above. Otherwise plain columns n0 + c.
    const int glu = p.glu_half;
    const int gshift = glu ? glu - BN / 2 : 0;
    const int m0 = tm * BM, n0 = tn * (glu ? BN / 2 : BN);

    // ---- this tile's panels and their valid extents in bytes (to the last
    // valid element of the operand)
    const char* a_panel = reinterpret_cast<const char*>(p.A + (int64_t)m0 * lda);
    const int64_t a_bytes = K > 0 ? (((int64_t)(M - 1) * lda + K) - (int64_t)m0 * lda) * 2 : 0;
    const char* b_panel = reinterpret_cast<const char*>(BCOL ? p.B + (int64_t)n0 * ldb : p.B + n0);
    const int64_t b_bytes = K <= 0 ? 0
                            : BCOL ? (((int64_t)(N - 1) * ldb + K) - (int64_t)n0 * ldb) * 2
                                   : (((int64_t)(K - 1) * ldb + N) - n0) * 2;
    // bytes between consecutive slabs in each panel
    const int64_t a_step = BK * 2;
    const int64_t b_step = BCOL ? BK * 2 : BK * ldb * 2;

    // ---- per-lane DMA source offsets (bytes), fixed for the whole K loop
    uint32_t voA[A_PER];
  #pragma unroll
    for (int t = 0; t < A_PER; ++t) {
      const int ins = wave + NW * t;
      const int r = 16 * ins + (lane >> 2);
      const int c = (lane & 3) ^ swzA(r);
      voA[t] = (uint32_t)(r * lda * 2) + c * 16;
    }
    const int b_cnt = (wave < B_DMA % NW) ? B_MAX : B_MIN;
    uint32_t voB[B_MAX];
  #pragma unroll
    for (int t = 0; t < B_MAX; ++t) {
      const int ins = wave + NW * t;
      if constexpr (BCOL) {
        const int r = 16 * ins + (lane >> 2);
        const int c = (lane & 3) ^ swzA(r);
        voB[t] = (uint32_t)((r + (r >= BN / 2 ? gshift : 0)) * ldb * 2) + c * 16;
      } else {
        const int q = 64 * ins + lane;
        const int row = q / CPR, pc = q - (q / CPR) * CPR;
        const int lc = SWB ? ((((pc >> 2) ^ (row & 3)) << 2) | (pc & 3)) : pc;
        voB[t] = (uint32_t)(row * ldb * 2) + lc * 16 + (lc >= CPR / 2 ? 2 * gshift : 0);
      }
    }

    const int nk = (K + BK - 1) / BK;
    // Slabs loaded by DMA; the rest (a K tail) go through registers. A buffer
    // load's range check works on whole dwords, so with a row-major B and an
    // odd N the dword holding B's last value (K - 1, N - 1) reaches past the
    // resource and would read as zero: the slab holding row K - 1 then takes
    // the masked register path too.
    const int nk_full = (!BCOL && (N & 1)) ? (K - 1) / BK : K / BK;

    // Issue the loads of slab s into its stage.
    auto issue_slab = [&](int s) {
      const int st = s % kStages;
      const uint32_t la = lds0 + st * STAGE;
      const uint32_t lb = la + A_BYTES;
      if (s < nk_full) {
        // the resources start at slab s (the range check then covers every
        // byte a lane reads; the scalar offset stays zero)
        const i32x4 rsA = make_rsrc(a_panel + s * a_step, a_bytes - s * a_step);
        const i32x4 rsB = make_rsrc(b_panel + s * b_step, b_bytes - s * b_step);
  #pragma unroll
        for (int t = 0; t < A_PER; ++t) dma16(la + 1024 * (wave + NW * t), rsA, voA[t], 0u);
  #pragma unroll
        for (int t = 0; t < B_MAX; ++t)
          if (t < B_MIN || t < b_cnt) dma16(lb + 1024 * (wave + NW * t), rsB, voB[t], 0u);
      } else {
        // K tail: exact zeros past K in both operands, through registers.
        const int k0 = s * BK;
        uint4* dA = reinterpret_cast<uint4*>(reinterpret_cast<char*>(smem) + st * STAGE);
        uint4* dB = reinterpret_cast<uint4*>(reinterpret_cast<char*>(smem) + st * STAGE + A_BYTES);
        for (int q = tid; q < BM * 4; q += NT) {
          const int r = q >> 2, c = q & 3;
          const uint4 v = (m0 + r < M) ? load8_masked(p.A + (int64_t)(m0 + r) * lda, k0 + 8 * c, K)
                                       : make_uint4(0, 0, 0, 0);
          dA[r * 4 + (c ^ swzA(r))] = v;
        }
        if constexpr (BCOL) {
          for (int q = tid; q < BN * 4; q += NT) {
            const int r = q >> 2, c = q & 3;
            const int col = n0 + r + (r >= BN / 2 ? gshift : 0);
            const uint4 v = (col < N) ? load8_masked(p.B + (int64_t)col * ldb, k0 + 8 * c, K)
                                      : make_uint4(0, 0, 0, 0);
            dB[r * 4 + (c ^ swzA(r))] = v;
          }
        } else {
          for (int q = tid; q < BK * CPR; q += NT) {
            const int row = q / CPR, pc = q - (q / CPR) * CPR;
            const int lc = SWB ? ((((pc >> 2) ^ (row & 3)) << 2) | (pc & 3)) : pc;
            const int gk = k0 + row;
            const int col = n0 + 8 * lc + (lc >= CPR / 2 ? gshift : 0);
            const uint4 v = (gk < K) ? load8_masked(p.B + (int64_t)gk * ldb, col, N)
                                     : make_uint4(0, 0, 0, 0);
            dB[row * CPR + pc] = v;
          }
        }
        wait_lgkmcnt0();
      }
    };

    // Issue DMA units [lo, hi) of full slab s: units 0 .. A_PER-1 are this
    // wave's A loads, then its b_cnt B loads.
    auto issue_units = [&](int s, int lo, int hi) {
      const uint32_t la = lds0 + (s % kStages) * STAGE;
      const uint32_t lb = la + A_BYTES;
      const i32x4 rsA = make_rsrc(a_panel + s * a_step, a_bytes - s * a_step);
      const i32x4 rsB = make_rsrc(b_panel + s * b_step, b_bytes - s * b_step);
  #pragma unroll
      for (int t = 0; t < A_PER; ++t)
        if (t >= lo && t < hi) dma16(la + 1024 * (wave + NW * t), rsA, voA[t], 0u);
  #pragma unroll
      for (int t = 0; t < B_MAX; ++t)
        if (t < b_cnt && A_PER + t >= lo && A_PER + t < hi) dma16(lb + 1024 * (wave + NW * t), rsB, voB[t], 0u);
    };

    // vmcnt waits are per wave. Wait until at most SLABS slabs' worth of this
    // wave's loads remain (waves < B_DMA % NW issue one more B load per slab).
    auto wait_slabs = [&](auto slabs_c) {
      constexpr int SL = decltype(slabs_c)::value;
      if (B_MAX != B_MIN && b_cnt == B_MAX)
        wait_vmcnt<SL * (A_PER + B_MAX)>();
      else
        wait_vmcnt<SL * (A_PER + B_MIN)>();
    };
    const std::integral_constant<int, 0> k0c{};
    const std::integral_constant<int, 1> k1c{};
    const std::integral_constant<int, 2> k2c{};

    floatx16 acc[FM][FN];
  #pragma unroll
    for (int i = 0; i < FM; ++i)
  #pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = floatx16{};

    const int lrow = lane & 31;
    const int lgrp = lane >> 5;
    // row-major B transposed reads: lane = 16 G + 4 j + q
    const int tG = lane >> 4, tj = (lane >> 2) & 3, tq = lane & 3;

    bf16x8 af[2][FM], bfr[2][FN];
    auto read_frags = [&](int s, int kk, int slot) {
      const uint32_t sbase = lds0 + (s % kStages) * STAGE;
      const int ch = 2 * kk + lgrp;
  #pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WTM + 32 * i + lrow;
        af[slot][i] = lds_read16(sbase + r * 64 + ((ch ^ swzA(r)) << 4));
      }
  #pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (BCOL) {
          const int r = wn * WTN + 32 * j + lrow;
          bfr[slot][j] = lds_read16(sbase + A_BYTES + r * 64 + ((ch ^ swzA(r)) << 4));
        } else {
          const int n = wn * WTN + 32 * j + 16 * (tG & 1) + 4 * tq;
          i16x4 h[2];
  #pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int row = 16 * kk + 8 * (tG >> 1) + 4 * t + tj;
            const int col = SWB ? ((((n >> 5) ^ (row & 3)) << 5) | (n & 31)) : n;
            h[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(uintptr_t)(sbase + A_BYTES + row * PITCH +
                                                                    col * 2));
          }
          bfr[slot][j] =
              __builtin_bit_cast(bf16x8, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
    };
    auto mfmas = [&](int slot) {
  #pragma unroll
      for (int i = 0; i < FM; ++i)
  #pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mma(af[slot][i], bfr[slot][j], acc[i][j]);
    };
    // Scheduling pattern for one 16-k step: each of the next step's operand
    // reads is issued right after one MFMA of this step, so reads overlap the
    // MFMAs and never pile up beyond what the LDS counter can track.
    constexpr int NREAD = FM + (BCOL ? FN : 2 * FN);
    constexpr int NMFMA = FM * FN;
    constexpr int RPM = (NREAD + NMFMA - 1) / NMFMA;  // reads issued after each MFMA
    auto interleave = [&]() {
  #pragma unroll
      for (int k = 0; k < NMFMA; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        if (k * RPM < NREAD) __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);  // LDS reads
      }
    };

    // The steady loop below spreads each slab's loads over two steps: the
    // first ceil(n/2) of a wave's n DMA units go out after the barrier of one
    // slab, the rest in the first step of the next, so the loads of a slab
    // never arrive at the texture unit faster than it drains them.
    const int n_steady = nk_full - (kStages - 1);  // slabs the steady loop may cover
    const bool split = n_steady >= kStages;        // the steady loop runs
    const int ndma = A_PER + b_cnt;
    const int nh1 = (ndma + 1) / 2;

    // ---- prologue: slabs 0..kStages-2 in flight (the last one only its first
    // half when the steady loop runs), slab 0 ready, its first operands read
    if (nk > 0) {
  #pragma unroll
      for (int s = 0; s < kStages - 1; ++s) {
        if (s < nk) {
          if (split && s == kStages - 2) issue_units(s, 0, nh1);
          else issue_slab(s);
        }
      }
      if (split) {
        // everything issued after slab 0: kStages-3 whole slabs and a first half
        if (B_MAX != B_MIN && b_cnt == B_MAX)
          wait_vmcnt<(kStages - 3) * (A_PER + B_MAX) + (A_PER + B_MAX + 1) / 2>();
        else
          wait_vmcnt<(kStages - 3) * (A_PER + B_MIN) + (A_PER + B_MIN + 1) / 2>();
      } else {
        const int after = nk - 1 < kStages - 2 ? nk - 1 : kStages - 2;
        if (after >= 4) wait_slabs(std::integral_constant<int, 4>{});
        else if (after == 3) wait_slabs(std::integral_constant<int, 3>{});
        else if (after == 2) wait_slabs(k2c);
        else if (after == 1) wait_slabs(k1c);
        else wait_slabs(k0c);
      }
      block_barrier();
      read_frags(0, 0, 0);
    }

    // ---- steady state: slabs whose slab-plus-3 is a full slab. No branches,
    // unrolled by the ring depth so every stage index is a compile-time
    // constant: LDS addresses are a lane register plus an immediate, DMA
    // destinations an SGPR plus a constant, and the buffer resources advance by
    // scalar adds.
    const int swl = (lrow >> 2) & 3;  // swzA of this lane's rows
    constexpr int NPAIR = (kStages + 1) / 2;  // stage pairs: one base register each
    uint32_t rA[2][NPAIR], rB[2][NPAIR];      // [kk][pair]: K-contiguous operands
  #pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint32_t chunk = (uint32_t)(((lgrp ^ swl) ^ (2 * kk)) << 4);
      const uint32_t a = lds0 + (wm * WTM + lrow) * 64 + chunk;
      const uint32_t b = lds0 + A_BYTES + (wn * WTN + lrow) * 64 + chunk;
  #pragma unroll
      for (int h = 0; h < NPAIR; ++h) {
        rA[kk][h] = a + 2 * h * STAGE;
        rB[kk][h] = b + 2 * h * STAGE;
      }
    }
    uint32_t rT[BCOL ? 1 : FN][NPAIR];        // row-major B: per block j and pair
  #pragma unroll
    for (int j = 0; j < (BCOL ? 1 : FN); ++j) {
      const int n = wn * WTN + 32 * j + 16 * (tG & 1) + 4 * tq;
      const int col = SWB ? ((((n >> 5) ^ tj) << 5) | (n & 31)) : n;
      const uint32_t b = lds0 + A_BYTES + (8 * (tG >> 1) + tj) * PITCH + col * 2;
  #pragma unroll
      for (int h = 0; h < NPAIR; ++h) rT[j][h] = b + 2 * h * STAGE;
    }
    const uint32_t ldsw = __builtin_amdgcn_readfirstlane(lds0 + 1024 * wave);

    // operand unit IDX of step KK from stage ST: A block IDX < FM, else B block
    auto read_fast = [&](auto st_c, auto kk_c, int slot, auto idx_c) {
      constexpr int ST = decltype(st_c)::value, KK = decltype(kk_c)::value;
      constexpr int IDX = decltype(idx_c)::value;
      constexpr int H = ST >> 1;
      constexpr uint32_t SO = (ST & 1) * STAGE;
      if constexpr (IDX < FM) {
        af[slot][IDX] = lds_read16(rA[KK][H] + (SO + IDX * 2048));
      } else if constexpr (BCOL) {
        bfr[slot][IDX - FM] = lds_read16(rB[KK][H] + (SO + (IDX - FM) * 2048));
      } else {
        constexpr int J = IDX - FM;
        const i16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(uintptr_t)(rT[J][H] + (SO + KK * 16 * PITCH)));
        const i16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(uintptr_t)(rT[J][H] +
                                                                (SO + KK * 16 * PITCH + 4 * PITCH)));
        bfr[slot][J] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    constexpr int NUNIT = FM + FN;
    constexpr int UPM = (NUNIT + NMFMA - 1) / NMFMA;  // operand units read after each MFMA
    constexpr int RPU = BCOL ? 1 : 2;                  // LDS read instructions per B unit
    // Hold the scheduler to "one MFMA, then that MFMA's share of the next
    // step's operand reads": left alone it sinks the reads below the MFMAs that
    // free their registers, and the next step then waits on LDS latency.
    auto pin_pattern = [&]() {
      static_for<0, NMFMA>([&](auto k_c) {
        constexpr int k = decltype(k_c)::value;
        constexpr int lo = k * UPM, hi = (k + 1) * UPM < NUNIT ? (k + 1) * UPM : NUNIT;
        constexpr int n_a = (lo < FM ? (hi < FM ? hi : FM) - lo : 0);
        constexpr int n_b = (hi > FM ? hi - (lo > FM ? lo : FM) : 0);
        constexpr int n_rd = lo < NUNIT ? n_a + RPU * n_b : 0;
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (n_rd > 0) __builtin_amdgcn_sched_group_barrier(0x100, n_rd, 0);
      });
    };

    auto steady = [&](auto bc_c) -> int {
      constexpr int BC = decltype(bc_c)::value;  // this wave's B loads per slab
      constexpr int NDMA = A_PER + BC;
      constexpr int NH1 = (NDMA + 1) / 2;        // units issued after a barrier
      constexpr int NH2 = NDMA - NH1;            // units issued one step later
      // Unit t of n goes out after MFMA (2t + 1) NMFMA / (2n) of its step: spread
      // evenly, so the waves' loads do not all reach the texture unit at once.
      auto dma_slot = [](int t, int n) constexpr { return ((2 * t + 1) * NMFMA) / (2 * n); };
      int s = 0;
      if (!split) return 0;
      // Unit U of the slab whose stage is STG, from resources rA_/rB_.
      auto unit = [&](auto stg_c, auto u_c, const i32x4& rA_, const i32x4& rB_) {
        constexpr int STG = decltype(stg_c)::value, U = decltype(u_c)::value;
        if constexpr (U < A_PER)
          dma16_off<STG * STAGE + 1024 * NW * U>(ldsw, rA_, voA[U]);
        else
          dma16_off<STG * STAGE + A_BYTES + 1024 * NW * (U - A_PER)>(ldsw, rB_, voB[U - A_PER]);
      };
      // resources of slab kStages-2, whose first half the prologue issued
      i32x4 rsAn = make_rsrc(a_panel + (kStages - 2) * a_step, a_bytes - (kStages - 2) * a_step);
      i32x4 rsBn = make_rsrc(b_panel + (kStages - 2) * b_step, b_bytes - (kStages - 2) * b_step);
      for (; s + kStages <= n_steady; s += kStages) {
        static_for<0, kStages>([&](auto st_c) {
          constexpr int ST = decltype(st_c)::value;         // stage of slab s + ST
          constexpr int STN = (ST + 1) % kStages;            // stage of slab s + ST + 1
          constexpr int STD = (ST + kStages - 1) % kStages;  // stage of slab s + ST + kStages - 1
          constexpr int ST2 = (ST + kStages - 2) % kStages;  // stage of slab s + ST + kStages - 2
          // MFMAs (slab, 0) while reading the operands of (slab, 1) and issuing
          // the second half of slab + kStages - 2 (its stage was freed by the
          // barrier of the previous slab)
          static_for<0, NMFMA>([&](auto k_c) {
            constexpr int k = decltype(k_c)::value;
            acc[k / FN][k % FN] = mma(af[0][k / FN], bfr[0][k % FN], acc[k / FN][k % FN]);
            static_for<0, UPM>([&](auto r_c) {
              constexpr int idx = k * UPM + decltype(r_c)::value;
              if constexpr (idx < NUNIT)
                read_fast(st_c, std::integral_constant<int, 1>{}, 1, std::integral_constant<int, idx>{});
            });
            static_for<0, NH2>([&](auto t_c) {
              constexpr int t = decltype(t_c)::value;
              if constexpr (dma_slot(t, NH2) == k)
                unit(std::integral_constant<int, ST2>{}, std::integral_constant<int, NH1 + t>{}, rsAn, rsBn);
            });
          });
          pin_pattern();
          advance_rsrc(rsAn, (uint32_t)a_step);
          advance_rsrc(rsBn, (uint32_t)b_step);
          // slab + 1 has landed once at most the loads issued after its last
          // half remain: halves of later slabs, kStages - 3 slabs' worth
          wait_vmcnt<(kStages - 3) * NDMA>();
          block_barrier();
          // MFMAs (slab, 1) while reading (slab + 1, 0) and issuing the first
          // half of slab + kStages - 1 into the stage the barrier just freed
          static_for<0, NMFMA>([&](auto k_c) {
            constexpr int k = decltype(k_c)::value;
            acc[k / FN][k % FN] = mma(af[1][k / FN], bfr[1][k % FN], acc[k / FN][k % FN]);
            static_for<0, UPM>([&](auto r_c) {
              constexpr int idx = k * UPM + decltype(r_c)::value;
              if constexpr (idx < NUNIT)
                read_fast(std::integral_constant<int, STN>{}, std::integral_constant<int, 0>{}, 0,
                          std::integral_constant<int, idx>{});
            });
            static_for<0, NH1>([&](auto t_c) {
              constexpr int t = decltype(t_c)::value;
              if constexpr (dma_slot(t, NH1) == k)
                unit(std::integral_constant<int, STD>{}, std::integral_constant<int, t>{}, rsAn, rsBn);
            });
          });
          pin_pattern();
        });
      }
      // The second half of slab s + kStages - 2 (stage kStages - 2, as s is a
      // multiple of kStages) is still due; after it every slab in flight is
      // whole again, which is what the general loop expects.
      static_for<0, NH2>([&](auto t_c) {
        unit(std::integral_constant<int, kStages - 2>{}, std::integral_constant<int, NH1 + decltype(t_c)::value>{},
             rsAn, rsBn);
      });
      return s;
    };
    int s0 = 0;
    if constexpr (B_MAX != B_MIN) {
      if (b_cnt == B_MAX) s0 = steady(std::integral_constant<int, B_MAX>{});
      else s0 = steady(std::integral_constant<int, B_MIN>{});
    } else {
      s0 = steady(std::integral_constant<int, B_MIN>{});
    }

    // ---- remaining slabs (and a K tail): the general loop
    for (int s = s0; s < nk; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      mfmas(0);
      read_frags(s, 1, 1);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      const bool more = s + 1 < nk;
      if (more) {
        // this wave's loads of slab s+1 are done once at most the loads of the
        // slabs issued after it remain (slabs s+2 .. s+kStages-2 that exist)
        const int after = (nk - 2 - s) < (kStages - 3) ? (nk - 2 - s) : (kStages - 3);
        if (after >= 3) wait_slabs(std::integral_constant<int, 3>{});
        else if (after == 2) wait_slabs(k2c);
        else if (after == 1) wait_slabs(k1c);
        else wait_slabs(k0c);
        block_barrier();
        if (s + kStages - 1 < nk) issue_slab(s + kStages - 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      mfmas(1);
      // unconditional so it can interleave with the MFMAs; after the last slab
      // it reads a stale stage (in bounds) whose values are never used
      read_frags(s + 1, 0, 0);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
    }

    // Epilogue: each accumulator element is stored exactly once, by its owner.
    // The K loop is over, so the LDS ring is free: each wave stages strips of
    // its sub-tile there (SH rows x WTN columns, row-major, padded rows) and
    // reads them back as 16-byte row chunks, so every global store writes whole
    // row segments instead of scattered 8- or 16-byte pieces.
    constexpr int ESZ = OUT_BF16 ? 2 : 4;
    constexpr int RING = kStages * STAGE;
    constexpr int OPITCH = WTN * ESZ + 16;  // staged row pitch (bytes); /16 is odd
    constexpr int SH = (NW * 32 * OPITCH <= RING) ? 32 : 16;
    static_assert(NW * SH * OPITCH <= RING, "a staged strip of every wave fits the ring");
    constexpr int CH = WTN * ESZ / 16;  // 16-byte chunks per staged row
    constexpr int EPC = 16 / ESZ;       // elements per chunk
    static_assert((SH * CH) % 64 == 0, "a strip is a whole number of wave-wide chunk rows");
    __syncthreads();  // every wave is done reading the ring
    if (glu) {
      // SiLU(gate) * up: a gate column and its up column sit in different
      // waves' sub-tiles, so every wave stages its strip of 32 (or 16) rows
      // into one block-wide fp32 strip, and after a barrier all threads form
      // silu(gate) * up for the BN/2 output columns and store them.
      constexpr int OPG = BN * 4 + 16;
      constexpr int SHG = (WM * 32 * OPG <= RING) ? 32 : 16;
      static_assert(WM * SHG * OPG <= RING, "a block-wide fp32 strip fits the ring");
      static_assert(BN / 2 % 8 == 0 && BN / 2 / 4 <= NT, "whole output chunks per block row");
      const EpiOut eo{p.C, p.ldc, M, glu, p.bias, p.act, p.counts, p.flags};
  #pragma unroll
      for (int i = 0; i < FM; ++i) {
  #pragma unroll
        for (int hs = 0; hs < 32 / SHG; ++hs) {
          const int rl = lrow - SHG * hs;
          if (SHG == 32 || (lrow >> 4) == hs) {
  #pragma unroll
            for (int j = 0; j < FN; ++j)
  #pragma unroll
              for (int q = 0; q < 4; ++q)
                lds_store_f4(lds0 + (uint32_t)((wm * SHG + rl) * OPG + (wn * WTN + 32 * j + 8 * q + 4 * lgrp) * 4),
                             floatx4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                     acc[i][j][4 * q + 3]});
          }
          __syncthreads();
          store_staged_glu<OUT_BF16, DEBUG>(lds0, OPG, WM * SHG, BN / 2, SHG, WTM,
                                            m0 + 32 * i + SHG * hs, n0, tid, NT, eo);
          __syncthreads();
        }
      }
      continue;
    }
    if (p.bias != nullptr || p.act != kActNone) {
      // Fused epilogue: strips are staged as fp32 whatever the output type and
      // read back by a rolled loop that adds the bias, applies the activation
      // and then converts, so the activation code is emitted once.
      constexpr int OPF = WTN * 4 + 16;
      constexpr int SHF = (NW * 32 * OPF <= RING) ? 32 : 16;
      static_assert(NW * SHF * OPF <= RING, "an fp32 strip of every wave fits the ring");
      static_assert(WTN / 4 <= 64, "one wave covers a staged row in 16-byte chunks");
      const uint32_t stf = lds0 + (uint32_t)(wave * SHF * OPF);
      const EpiOut eo{p.C, p.ldc, M, N, p.bias, p.act, p.counts, p.flags};
  #pragma unroll
      for (int i = 0; i < FM; ++i) {
  #pragma unroll
        for (int hs = 0; hs < 32 / SHF; ++hs) {
          const int rl = lrow - SHF * hs;
          if (SHF == 32 || (lrow >> 4) == hs) {
  #pragma unroll
            for (int j = 0; j < FN; ++j)
  #pragma unroll
              for (int q = 0; q < 4; ++q)
                lds_store_f4(stf + (uint32_t)(rl * OPF + (32 * j + 8 * q + 4 * lgrp) * 4),
                             floatx4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                     acc[i][j][4 * q + 3]});
          }
          wait_lgkmcnt0();
          store_staged_fused<OUT_BF16, DEBUG>(stf, OPF, SHF, WTN, m0 + wm * WTM + 32 * i + SHF * hs,
                                              n0 + wn * WTN, lane, 64, eo);
          wait_lgkmcnt0();
        }
      }
      wait_lgkmcnt0();
      block_barrier();
      continue;
    }
    const uint32_t stg = lds0 + (uint32_t)(wave * SH * OPITCH);
    const bool full_mn = (m0 + BM <= M) && (n0 + BN <= N);
  #pragma unroll
    for (int i = 0; i < FM; ++i) {
  #pragma unroll
      for (int hs = 0; hs < 32 / SH; ++hs) {
        // lane l holds row (l % 32) of the block and, for q = 0..3, the four
        // consecutive columns 8 q + 4 (l / 32) .. + 3 (accumulator 4 q .. 4 q + 3)
        const int rl = lrow - SH * hs;
        if (SH == 32 || (lrow >> 4) == hs) {
  #pragma unroll
          for (int j = 0; j < FN; ++j) {
  #pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t a = stg + (uint32_t)(rl * OPITCH + (32 * j + 8 * q + 4 * lgrp) * ESZ);
              const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1];
              const float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
              if constexpr (OUT_BF16) {
                const u32x2v w = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
                *(__attribute__((address_space(3))) u32x2v*)(uintptr_t)a = w;
              } else {
                const floatx4 w = {v0, v1, v2, v3};
                *(__attribute__((address_space(3))) floatx4*)(uintptr_t)a = w;
              }
            }
          }
        }
        // The strip is private to this wave and one wave's LDS operations run
        // in order, so its reads below see its writes above.
        wait_lgkmcnt0();
        const int grow0 = m0 + wm * WTM + 32 * i + SH * hs;
        const int gcol0 = n0 + wn * WTN;
  #pragma unroll
        for (int c0 = 0; c0 < SH * CH; c0 += 64) {
          const int c = c0 + lane;
          const int r = c / CH, ch = c - (c / CH) * CH;
          const u32x4v lv = *(const __attribute__((address_space(3))) u32x4v*)(uintptr_t)(stg + (uint32_t)(r * OPITCH + ch * 16));
          const uint4 v = make_uint4(lv.x, lv.y, lv.z, lv.w);
          const int row = grow0 + r, col = gcol0 + ch * EPC;
          const int64_t off = (int64_t)row * p.ldc + col;
          char* cbase = static_cast<char*>(p.C) + off * ESZ;
          if (full_mn || (row < M && col + EPC <= N)) {
            *reinterpret_cast<uint4*>(cbase) = v;
            if constexpr (DEBUG) {
              if (p.flags & kDbgCount)
  #pragma unroll
                for (int e = 0; e < EPC; ++e) atomicAdd(p.counts + (int64_t)row * N + col + e, 1u);
            }
          } else if (row < M) {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  #pragma unroll
            for (int e = 0; e < EPC; ++e) {
              if (col + e < N) {
                if constexpr (OUT_BF16) {
                  reinterpret_cast<uint16_t*>(cbase)[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
                } else {
                  reinterpret_cast<uint32_t*>(cbase)[e] = w[e];
                }
                if constexpr (DEBUG) {
                  if (p.flags & kDbgCount) atomicAdd(p.counts + (int64_t)row * N + col + e, 1u);
                }
              }
            }
          }
        }
        wait_lgkmcnt0();
      }
    }
    // The next tile's loads reuse the ring: every wave must be done reading
    // its staged strips (the stores may still be in flight).
    wait_lgkmcnt0();
    block_barrier();
  }
}

}  // namespace tg
