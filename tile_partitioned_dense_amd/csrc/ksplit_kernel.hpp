// ksplit_kernel.hpp -- the tile kernel for small tiles with K split across
// the waves of one workgroup, for shapes whose tiles are too few or too small
// to keep the chip busy with one K walk per tile (tall-skinny outputs such as
// 4096 x 256 with K = 4096).
//
// Ownership is unchanged: every BM x BN tile has exactly one owning workgroup
// (tile_of, tiles w, w + grid, ...), which is its only writer. Inside the
// workgroup, wave w multiplies the whole tile over its own contiguous range
// of 32-wide K slabs, in ascending order, through a ring of LDS buffers that
// only it fills and reads -- so the K loop needs no barrier across waves.
// The waves' partial tiles then meet in LDS along a fixed pairwise tree (wave
// w adds wave w + h for h = KS/2, ..., 1), the same fixed-order combine as
// the decode kernel and the fixed-order workgroup reductions of "Rust Compute
// Kernels" (section "Signature mapping"); wave 0 stores the tile. The split
// points depend only on K and KS, so every element's summation order is fixed
// and results are bit-identical from run to run. There is no atomic and no
// second writer.
//
// Operand staging, LDS layouts, MFMA operand reads and the transposed
// accumulator layout are those of the tile kernel (tile_kernel.hpp), per wave.
#pragma once

#include "tile_kernel.hpp"

namespace tg {

template <int BM, int BN, int KS, int NST, bool BCOL, bool OUT_BF16, bool DEBUG>
__global__ __launch_bounds__(KS * 64, 1) void ksplit_gemm_kernel(TileArgs p) {
  static_assert(KS == 2 || KS == 4 || KS == 8, "pairwise tree needs a power of two");
  static_assert(NST >= 2 && NST <= 8, "ring depth");
  constexpr int FM = BM / 32, FN = BN / 32;
  static_assert(BM % 32 == 0 && BN % 32 == 0, "tile must be a multiple of 32");
  constexpr int BK = kTileBK;
  constexpr int A_BYTES = BM * BK * 2;  // per slab
  constexpr int B_BYTES = BN * BK * 2;
  constexpr int SLAB = A_BYTES + B_BYTES;
  constexpr int RING = NST * SLAB;  // per wave
  constexpr int A_UNITS = A_BYTES / 1024, B_UNITS = B_BYTES / 1024;
  static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "slabs are whole KiB");
  constexpr int PITCH = BN * 2;  // row-major B: bytes per k row
  constexpr bool SWB = !BCOL && (PITCH % 256 == 0);
  constexpr int CPR = BN / 8;    // row-major B: 16-byte chunks per k row
  constexpr int RED = (KS / 2) * BM * BN * 4;  // partial tiles in flight in the tree
  constexpr int LDS = (KS * RING > RED) ? KS * RING : RED;

  __shared__ __attribute__((aligned(1024))) uint4 smem[LDS / 16];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t ring = lds0 + (uint32_t)(wave * RING);
  const int M = p.M, N = p.N, K = p.K;
  const int64_t lda = p.lda, ldb = p.ldb;
  // SiLU(gate) * up: the tile's last BN/2 columns are the up columns of its
  // first BN/2 gate columns (B column shift glu - BN/2), as in the tile kernel
  const int glu = p.glu_half;
  const int gshift = glu ? glu - BN / 2 : 0;
  const int lrow = lane & 31, lgrp = lane >> 5;
  const int tG = lane >> 4, tj = (lane >> 2) & 3, tq = lane & 3;

  // this wave's K range, in slabs
  const int nk = (K + BK - 1) / BK;
  // DMA slabs; with a row-major B and an odd N the slab holding row K - 1
  // goes through the register path, as in the tile kernel (a buffer load
  // zeroes the dword that straddles the end of B, which holds its last value)
  const int nk_full = (!BCOL && (N & 1)) ? (K - 1) / BK : K / BK;
  const int kb0 = (wave * nk) / KS, kb1 = ((wave + 1) * nk) / KS;

  // per-lane DMA source offsets within a slab (bytes), as in the tile kernel
  uint32_t voA[A_UNITS], voB[B_UNITS];
#pragma unroll
  for (int u = 0; u < A_UNITS; ++u) {
    const int r = 16 * u + (lane >> 2);
    voA[u] = (uint32_t)(r * lda * 2) + (((lane & 3) ^ swzA(r)) << 4);
  }
#pragma unroll
  for (int u = 0; u < B_UNITS; ++u) {
    if constexpr (BCOL) {
      const int r = 16 * u + (lane >> 2);
      voB[u] = (uint32_t)((r + (r >= BN / 2 ? gshift : 0)) * ldb * 2) + (((lane & 3) ^ swzA(r)) << 4);
    } else {
      const int q = 64 * u + lane;
      const int row = q / CPR, pc = q - (q / CPR) * CPR;
      const int lc = SWB ? ((((pc >> 2) ^ (row & 3)) << 2) | (pc & 3)) : pc;
      voB[u] = (uint32_t)(row * ldb * 2) + lc * 16 + (lc >= CPR / 2 ? 2 * gshift : 0);
    }
  }
  const uint32_t ldsw = __builtin_amdgcn_readfirstlane(ring);

  const int n_tiles = p.map.tiles_m * p.map.tiles_n;
  for (int wg_it = blockIdx.x; wg_it < n_tiles; wg_it += gridDim.x) {
    int wg = wg_it;
    if constexpr (DEBUG) {
      if ((p.flags & kDbgCollide) && wg == 1) wg = 0;  // negative control only
    }
    int32_t tm, tn;
    tile_of(p.map, wg, tm, tn);
    const int m0 = tm * BM, n0 = tn * (glu ? BN / 2 : BN);
    const char* a_panel = reinterpret_cast<const char*>(p.A + (int64_t)m0 * lda);
    const int64_t a_bytes = K > 0 ? (((int64_t)(M - 1) * lda + K) - (int64_t)m0 * lda) * 2 : 0;
    const char* b_panel = reinterpret_cast<const char*>(BCOL ? p.B + (int64_t)n0 * ldb : p.B + n0);
    const int64_t b_bytes = K <= 0 ? 0
                            : BCOL ? (((int64_t)(N - 1) * ldb + K) - (int64_t)n0 * ldb) * 2
                                   : (((int64_t)(K - 1) * ldb + N) - n0) * 2;
    const int64_t a_step = BK * 2;
    const int64_t b_step = BCOL ? BK * 2 : BK * ldb * 2;

    // Load slab s into its stage of this wave's ring.
    auto issue_slab = [&](int s) {
      const int st = s % NST;
      const uint32_t la = ldsw + st * SLAB;
      if (s < nk_full) {
        const i32x4 rsA = make_rsrc(a_panel + s * a_step, a_bytes - s * a_step);
        const i32x4 rsB = make_rsrc(b_panel + s * b_step, b_bytes - s * b_step);
#pragma unroll
        for (int u = 0; u < A_UNITS; ++u) dma16(la + 1024 * u, rsA, voA[u], 0u);
#pragma unroll
        for (int u = 0; u < B_UNITS; ++u) dma16(la + A_BYTES + 1024 * u, rsB, voB[u], 0u);
      } else {
        // K tail: exact zeros past K in both operands, through registers
        const int k0 = s * BK;
        uint4* dA = reinterpret_cast<uint4*>(reinterpret_cast<char*>(smem) + wave * RING + st * SLAB);
        uint4* dB = reinterpret_cast<uint4*>(reinterpret_cast<char*>(smem) + wave * RING + st * SLAB + A_BYTES);
        for (int q = lane; q < BM * 4; q += 64) {
          const int r = q >> 2, c = q & 3;
          const uint4 v = (m0 + r < M) ? load8_masked(p.A + (int64_t)(m0 + r) * lda, k0 + 8 * c, K)
                                       : make_uint4(0, 0, 0, 0);
          dA[r * 4 + (c ^ swzA(r))] = v;
        }
        if constexpr (BCOL) {
          for (int q = lane; q < BN * 4; q += 64) {
            const int r = q >> 2, c = q & 3;
            const int col = n0 + r + (r >= BN / 2 ? gshift : 0);
            const uint4 v = (col < N) ? load8_masked(p.B + (int64_t)col * ldb, k0 + 8 * c, K)
                                      : make_uint4(0, 0, 0, 0);
            dB[r * 4 + (c ^ swzA(r))] = v;
          }
        } else {
          for (int q = lane; q < BK * CPR; q += 64) {
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
    // wait until at most `after` slabs' DMA loads of this wave are pending
    auto wait_after = [&](int after) {
      constexpr int U = A_UNITS + B_UNITS;
      switch (after) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<(1 * U < 63 ? 1 * U : 63)>(); break;
        case 2: wait_vmcnt<(2 * U < 63 ? 2 * U : 63)>(); break;
        case 3: wait_vmcnt<(3 * U < 63 ? 3 * U : 63)>(); break;
        case 4: wait_vmcnt<(4 * U < 63 ? 4 * U : 63)>(); break;
        case 5: wait_vmcnt<(5 * U < 63 ? 5 * U : 63)>(); break;
        default: wait_vmcnt<(6 * U < 63 ? 6 * U : 63)>(); break;
      }
    };

    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = floatx16{};

    for (int s = kb0; s < kb0 + NST - 1 && s < kb1; ++s) issue_slab(s);
    for (int s = kb0; s < kb1; ++s) {
      // The stage of slab s - 1 takes slab s + NST - 1: this wave's reads of
      // it have returned (waited for here, not only implied by the MFMAs).
      const int nxt = s + NST - 1;
      wait_lgkmcnt0();
      if (nxt < kb1) issue_slab(nxt);
      // Slab s has landed once at most the DMA loads of the slabs issued
      // after it remain. A K-tail slab (always the last) is read through
      // registers and complete when issued, so it does not count.
      const int last = (nxt < kb1 ? nxt : kb1 - 1);
      const int after = last - s - ((last > s && last >= nk_full) ? 1 : 0);
      wait_after(after > 6 ? 6 : after);
      asm volatile("" ::: "memory");
      const uint32_t sb = ldsw + (s % NST) * SLAB;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 af[FM], bfr[FN];
        const int ch = 2 * kk + lgrp;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = 32 * i + lrow;
          af[i] = lds_read16(sb + r * 64 + ((ch ^ swzA(r)) << 4));
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if constexpr (BCOL) {
            const int r = 32 * j + lrow;
            bfr[j] = lds_read16(sb + A_BYTES + r * 64 + ((ch ^ swzA(r)) << 4));
          } else {
            const int n = 32 * j + 16 * (tG & 1) + 4 * tq;
            i16x4 h[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const int row = 16 * kk + 8 * (tG >> 1) + 4 * t + tj;
              const int col = SWB ? ((((n >> 5) ^ (row & 3)) << 5) | (n & 31)) : n;
              h[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) i16x4*)(uintptr_t)(sb + A_BYTES + row * PITCH + col * 2));
            }
            bfr[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
          }
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mma(af[i], bfr[j], acc[i][j]);
      }
    }

    // Fixed pairwise tree over the waves' partial tiles (the K loops and
    // their LDS reads are over once every wave reaches the barrier).
    __syncthreads();
    floatx16* red = reinterpret_cast<floatx16*>(smem);  // [KS/2][FM*FN][64]
#pragma unroll
    for (int h = KS / 2; h >= 1; h >>= 1) {
      if (wave >= h && wave < 2 * h) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) red[((wave - h) * FM * FN + i * FN + j) * 64 + lane] = acc[i][j];
      }
      __syncthreads();
      if (wave < h) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] += red[(wave * FM * FN + i * FN + j) * 64 + lane];
      }
      __syncthreads();
    }

    if (p.bias != nullptr || p.act != kActNone) {
      // Fused epilogue: wave 0 stages the summed tile as fp32 rows in LDS and
      // every wave takes a share of the bias / activation / store pass, one
      // rolled loop (the activation code is emitted once).
      constexpr int OPF = BN * 4 + 16;
      static_assert(BM * OPF <= LDS, "the fp32 tile fits the workgroup's LDS");
      static_assert(BN / 4 <= KS * 64, "the workgroup covers a staged row in 16-byte chunks");
      if (wave == 0) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              lds_store_f4(lds0 + (uint32_t)((32 * i + lrow) * OPF + (32 * j + 8 * q + 4 * lgrp) * 4),
                           floatx4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                   acc[i][j][4 * q + 3]});
      }
      __syncthreads();
      if (glu) {
        static_assert(BN / 2 % 8 == 0, "whole output chunks per row");
        const EpiOut eo{p.C, p.ldc, M, glu, p.bias, p.act, p.counts, p.flags};
        store_staged_glu<OUT_BF16, DEBUG>(lds0, OPF, BM, BN / 2, BM, 0, m0, n0, threadIdx.x,
                                          KS * 64, eo);
      } else {
        const EpiOut eo{p.C, p.ldc, M, N, p.bias, p.act, p.counts, p.flags};
        store_staged_fused<OUT_BF16, DEBUG>(lds0, OPF, BM, BN, m0, n0, threadIdx.x, KS * 64, eo);
      }
      __syncthreads();
      continue;
    }

    // Wave 0 stores the tile: lane l holds row (l % 32) of each 32 x 32 block
    // and, for q = 0..3, its four consecutive columns 8 q + 4 (l / 32) .. + 3.
    if (wave == 0) {
      const bool full_mn = (m0 + BM <= M) && (n0 + BN <= N);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = m0 + 32 * i + lrow;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = n0 + 32 * j + 8 * q + 4 * lgrp;
            const int64_t off = (int64_t)row * p.ldc + col;
            const float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                acc[i][j][4 * q + 3]};
            if (full_mn || (row < M && col + 3 < N)) {
              if constexpr (OUT_BF16) {
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.C) + off) =
                    make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
              } else {
                *reinterpret_cast<float4*>(static_cast<float*>(p.C) + off) = make_float4(v[0], v[1], v[2], v[3]);
              }
              if constexpr (DEBUG) {
                if (p.flags & kDbgCount)
#pragma unroll
                  for (int e = 0; e < 4; ++e) atomicAdd(p.counts + (int64_t)row * N + col + e, 1u);
              }
            } else if (row < M) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if (col + e < N) {
                  if constexpr (OUT_BF16) {
                    static_cast<uint16_t*>(p.C)[off + e] = f32_to_bf16(v[e]);
                  } else {
                    static_cast<float*>(p.C)[off + e] = v[e];
                  }
                  if constexpr (DEBUG) {
                    if (p.flags & kDbgCount) atomicAdd(p.counts + (int64_t)row * N + col + e, 1u);
                  }
                }
              }
            }
          }
        }
      }
    }
    // the next tile's loads reuse the rings the tree just used
    __syncthreads();
  }
}

}  // namespace tg
