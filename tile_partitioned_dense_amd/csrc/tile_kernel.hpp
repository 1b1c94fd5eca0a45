// tile_kernel.hpp -- the LDS-staged bf16 MFMA tile kernel for gfx950.
//
// One workgroup owns one BM x BN tile of C (found with tile_of) and is its
// only writer. It walks K in 64-wide slabs in ascending order:
//   global -> registers -> LDS (double-buffered: slab s+1 is fetched while slab
//   s is multiplied) -> MFMA operands -> fp32 accumulators,
// then stores its tile once. A and B are only read, so fetching ahead is
// always legal; C is never read.
//
// LDS layout: each slab row (64 bf16 = 128 bytes) is eight 16-byte chunks,
// and chunk c of row r is stored at position c ^ swz(r), swz(r) = (r ^ (r >> 3))
// & 7. MFMA operand reads (32 consecutive rows, one chunk) and the stores of
// both the row-major copy and the transposed copy (8 rows apart) then touch
// eight different chunk positions per group of eight lanes.
//
// Both MFMA operands want 8 consecutive k values per lane. A is K-contiguous;
// so is a column-major B. A row-major B is transposed in registers: a thread
// loads an 8 (k) x 8 (n) block as eight 16-byte rows and regroups the halves
// into eight 8-k columns before storing them.
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
};

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

template <int BM, int BN, int WM, int WN, bool BCOL, bool OUT_BF16, bool DEBUG>
__global__ __launch_bounds__(WM * WN * 64, 1) void tile_gemm_kernel(TileArgs p) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  constexpr int A_CH = BM * 8;  // 16-byte chunks per A slab
  constexpr int B_CH = BN * 8;
  static_assert(A_CH % NT == 0, "A slab must split evenly over the threads");
  constexpr int A_PER = A_CH / NT;
  static_assert(!BCOL || B_CH % NT == 0, "B slab must split evenly over the threads");
  constexpr int BC_PER = BCOL ? B_CH / NT : 1;        // column-major B: chunks per thread
  constexpr int BR_BLK = (BN + NT - 1) / NT;          // row-major B: 8x8 blocks per thread
  constexpr int BR_NB = BN / 8;                       // 8-column groups per slab row

  __shared__ uint4 smem[2 * (A_CH + B_CH)];
  uint4* const sA = smem;
  uint4* const sB = smem + 2 * A_CH;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave - (wave / WN) * WN;

  int wg = blockIdx.x;
  if constexpr (DEBUG) {
    if ((p.flags & kDbgCollide) && wg == 1) wg = 0;  // negative control only
  }
  int32_t tm, tn;
  tile_of(p.map, wg, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int M = p.M, N = p.N, K = p.K;
  const bool full_mn = (m0 + BM <= M) && (n0 + BN <= N);

  // Per-thread global source rows (64-bit offsets, formed once).
  const int a_r0 = tid >> 3, a_c = tid & 7;  // chunk (row, col) for pass 0
  constexpr int A_ROW_STEP = NT / 8;          // rows between passes
  const uint16_t* const a_base = p.A + (int64_t)(m0 + a_r0) * p.lda + 8 * a_c;

  uint4 ra[A_PER];
  uint4 rb[BCOL ? BC_PER : 8 * BR_BLK];

  // Fetch one K slab into registers. FAST (a compile-time constant) means the
  // whole slab is in range: plain vector loads with no per-load branches, so
  // every load of the slab is in flight at once. Otherwise rows are clamped
  // into range (the value is then replaced by zero) and the K / N tail of a
  // chunk is read element by element.
  auto load_slab = [&](int k0, auto fast_c) {
    constexpr bool FAST = decltype(fast_c)::value;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const uint16_t* src = a_base + (int64_t)i * A_ROW_STEP * p.lda;
      if constexpr (FAST) {
        ra[i] = *reinterpret_cast<const uint4*>(src + k0);
      } else {
        const int gm = m0 + a_r0 + i * A_ROW_STEP;
        const uint4 v = (gm < M) ? load8_masked(src - 8 * a_c, k0 + 8 * a_c, K) : make_uint4(0, 0, 0, 0);
        ra[i] = v;
      }
    }
    if constexpr (BCOL) {
#pragma unroll
      for (int i = 0; i < BC_PER; ++i) {
        const int q = i * NT + tid;
        const int r = q >> 3, c = q & 7;
        const uint16_t* src = p.B + (int64_t)(n0 + r) * p.ldb + 8 * c;
        if constexpr (FAST) {
          rb[i] = *reinterpret_cast<const uint4*>(src + k0);
        } else {
          rb[i] = (n0 + r < N) ? load8_masked(src - 8 * c, k0 + 8 * c, K) : make_uint4(0, 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < BR_BLK; ++i) {
        const int q = i * NT + tid;
        if (BN % NT == 0 || q < BN) {
          const int kb = q / BR_NB, nb = q - (q / BR_NB) * BR_NB;
          const int gc = n0 + 8 * nb;
#pragma unroll
          for (int rr = 0; rr < 8; ++rr) {
            const int gk = k0 + 8 * kb + rr;
            const uint16_t* src = p.B + (int64_t)gk * p.ldb;
            if constexpr (FAST) {
              rb[8 * i + rr] = *reinterpret_cast<const uint4*>(src + gc);
            } else {
              rb[8 * i + rr] = (gk < K) ? load8_masked(src, gc, N) : make_uint4(0, 0, 0, 0);
            }
          }
        }
      }
    }
  };

  auto store_slab = [&](int buf) {
    uint4* const dA = sA + buf * A_CH;
    uint4* const dB = sB + buf * B_CH;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int r = a_r0 + i * A_ROW_STEP;
      dA[r * 8 + (a_c ^ swz(r))] = ra[i];
    }
    if constexpr (BCOL) {
#pragma unroll
      for (int i = 0; i < BC_PER; ++i) {
        const int q = i * NT + tid;
        const int r = q >> 3, c = q & 7;
        dB[r * 8 + (c ^ swz(r))] = rb[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < BR_BLK; ++i) {
        const int q = i * NT + tid;
        if (BN % NT == 0 || q < BN) {
          const int kb = q / BR_NB, nb = q - (q / BR_NB) * BR_NB;
          // rb[8i + rr] holds columns 8nb..8nb+7 of k row 8kb+rr; column c
          // is dword c/2, half c%2. Regroup into column-major 8-k chunks.
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const bool hi = (c & 1) != 0;
            uint32_t w[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              const uint4& x = rb[8 * i + 2 * d];
              const uint4& y = rb[8 * i + 2 * d + 1];
              const uint32_t xs = (c >> 1) == 0 ? x.x : (c >> 1) == 1 ? x.y : (c >> 1) == 2 ? x.z : x.w;
              const uint32_t ys = (c >> 1) == 0 ? y.x : (c >> 1) == 1 ? y.y : (c >> 1) == 2 ? y.z : y.w;
              w[d] = pack_halves(xs, ys, hi);
            }
            const int n = 8 * nb + c;
            dB[n * 8 + (kb ^ swz(n))] = make_uint4(w[0], w[1], w[2], w[3]);
          }
        }
      }
    }
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx16{};

  const int lrow = lane & 31;
  const int lgrp = lane >> 5;

  // Multiply one staged slab: four 16-k steps; the operands of step kk+1 are
  // read from LDS while the MFMAs of step kk run.
  auto compute_slab = [&](int buf) {
    const uint4* const cA = sA + buf * A_CH;
    const uint4* const cB = sB + buf * B_CH;
    bf16x8 af[2][FM], bfr[2][FN];
    auto read_frags = [&](int kk, int slot) {
      const int ch = 2 * kk + lgrp;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WTM + 32 * i + lrow;
        af[slot][i] = as_bf16x8(cA[r * 8 + (ch ^ swz(r))]);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = wn * WTN + 32 * j + lrow;
        bfr[slot][j] = as_bf16x8(cB[n * 8 + (ch ^ swz(n))]);
      }
    };
    read_frags(0, 0);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      if (kk + 1 < kBK / 16) read_frags(kk + 1, (kk + 1) & 1);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32(af[kk & 1][i], bfr[kk & 1][j], acc[i][j]);
    }
  };

  const std::integral_constant<bool, true> kFast{};
  const std::integral_constant<bool, false> kMasked{};
  const int nk = (K + kBK - 1) / kBK;
  // slabs [0, nk_fast) need no masking: interior tile and K fully covered
  const int nk_fast = full_mn ? K / kBK : 0;

  if (nk > 0) {
    if (nk_fast > 0) load_slab(0, kFast);
    else load_slab(0, kMasked);
    store_slab(0);
  }
  __syncthreads();

  int s = 0;
  // steady state: the next slab is complete, so its loads are branch-free
  // (the scheduling barriers keep the compiler from sinking the loads of
  // slab s+1 below the MFMAs of slab s, which would expose their latency)
  for (; s + 1 < nk_fast; ++s) {
    load_slab((s + 1) * kBK, kFast);
    __builtin_amdgcn_sched_barrier(0);
    compute_slab(s & 1);
    __builtin_amdgcn_sched_barrier(0);
    store_slab((s & 1) ^ 1);
    __syncthreads();
  }
  for (; s < nk; ++s) {
    const bool more = (s + 1) < nk;
    if (more) load_slab((s + 1) * kBK, kMasked);
    __builtin_amdgcn_sched_barrier(0);
    compute_slab(s & 1);
    __builtin_amdgcn_sched_barrier(0);
    if (more) store_slab((s & 1) ^ 1);
    __syncthreads();
  }

  // Epilogue: each accumulator element is stored exactly once, by its owner.
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * WTN + 32 * j + lrow;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * WTM + 32 * i + 8 * (v >> 2) + 4 * lgrp + (v & 3);
        if (full_mn || (row < M && col < N)) {
          const int64_t off = (int64_t)row * p.ldc + col;
          if constexpr (OUT_BF16) {
            static_cast<uint16_t*>(p.C)[off] = f32_to_bf16_rne(acc[i][j][v]);
          } else {
            static_cast<float*>(p.C)[off] = acc[i][j][v];
          }
          if constexpr (DEBUG) {
            if (p.flags & kDbgCount) atomicAdd(p.counts + (int64_t)row * N + col, 1u);
          }
        }
      }
    }
  }
}

}  // namespace tg
