// stream_kernel.hpp -- bf16 product for few-row outputs with a column-major
// (K-contiguous) B, the layout in which weights are usually stored: the
// weight stream of a decode step, bound by HBM.
//
// Ownership is the tile kernel's: every BM x BN tile of C (BM = 16, 32 or
// 64 rows, so one tile row covers a decode batch) is owned by one workgroup,
// which reads A and B as shared immutable views and writes its tile once; a
// persistent grid walks tiles wg, wg + grid, ... (tile_of).
//
// K moves in stages of SB bytes (SB / 2 values) of every row of A and of B's
// columns, loaded straight into LDS (buffer loads with the lds modifier,
// through range-checked resources) so that each one-KiB load instruction
// covers 1024 / SB B columns with whole 128-byte lines; the tile kernel's
// 64-byte slab would cover sixteen columns with half a line each. In LDS a
// stage row is SB / 16 chunks of 16 bytes (8 values), chunk c of row r at
// position c ^ swz(r) (swz(r) = r & 15 for rows of 256 bytes or more,
// (r >> 1) & 7 for 128-byte rows), which the loads produce by permuting which chunk each lane
// fetches; the sixteen rows one MFMA operand read touches (same chunk,
// consecutive rows) then sit in sixteen distinct bank groups.
//
// KS waves (one or two) work on each 32-column block of the tile, all its
// rows: wave w takes block w % (BN / 32) and, of every stage's MFMA steps,
// the share (w / (BN / 32)) * NSTEP / KS ..; every wave issues a share of
// the loads (two waves per SIMD hide each other's issue stalls). A wave holds
// one 32 x 32 accumulator block per 32 rows, transposed (the B fragment is
// the MFMA's first operand, as in mma(), and is read once for all blocks),
// fed by v_mfma_f32_32x32x16_bf16 over chunk pairs 2 t, 2 t + 1 of a stage.
// With KS = 2 the second wave of a block adds its partial sums into the
// first's after the K loop, always in that order, and the first stores. With
// BM = 16 the lanes of rows 16..31 give zero A operands and are never
// stored.
//
// Each step waits for stage s, passes one barrier (after which every wave is
// done with stage s - 1), loads stage s + NST - 1 into stage s - 1's buffer
// and then runs stage s's MFMAs. Stages are numbered on across a workgroup's
// tiles (buffer (g + s) % NST, g the stages of its earlier tiles), so the
// last steps of a tile load the first stages of the workgroup's next tile
// and the next tile starts with its ring already filling; the store stages
// the tile in the buffer of its last stage, the one buffer no load is
// filling then. Each wave accumulates its share of K in
// ascending order in fp32, and the two shares of a block meet in a fixed
// order: results are bit-identical run to run. A last stage that ends
// inside K zeroes, in both operands, every value at or past K (the bytes
// loaded there belong to the next row, or read as zero past the operand).
// K must be even: the range check of a buffer load works on whole dwords, so
// with odd K the dword holding value K - 1 of an operand's last row reaches
// past the resource and reads as zero.
//
// SiLU(gate) * up (glu_half = N / 2): the tile's first BN / 2 columns are gate
// columns n0 .. and its last BN / 2 the up columns N / 2 + n0 .. (the loads
// shift the upper half of the B rows); the waves stage one block-wide fp32
// strip and all threads form silu(gate) * up for the BN / 2 output columns.
#pragma once

#include "tile_kernel.hpp"

namespace tg {

// Zero the values of a 16-byte chunk (8 bf16, lowest address first) from
// index `valid` on.
__device__ __forceinline__ bf16x8 keep_first(const bf16x8& v, int valid) {
  if (valid >= 8) return v;
  uint4 u = __builtin_bit_cast(uint4, v);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (2 * e >= valid) w[e] = 0u;
    else if (2 * e + 1 >= valid) w[e] &= 0xffffu;
  }
  return __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
}

template <int BM, int BN, int SB, int NST, int KS, bool OUT_BF16, bool DEBUG>
__global__ __launch_bounds__(BN / 32 * KS * 64, 1) void stream_gemm_kernel(TileArgs p) {
  static_assert(BM == 16 || BM == 32 || BM == 64, "half a 32-row block, or one or two blocks");
  static_assert(BN % 64 == 0 && BN <= 256, "whole waves, even gate and up halves");
  static_assert(SB == 128 || SB == 256 || SB == 512, "stage rows of whole 128-byte lines");
  static_assert(KS == 1 || KS == 2, "one or two waves per 32-column block");
  constexpr int NCB = BN / 32;               // 32-column blocks
  constexpr int NW = NCB * KS;               // waves (all of them issue loads)
  constexpr int NT = NW * 64;
  constexpr int FM = BM < 32 ? 1 : BM / 32;   // 32-row accumulator blocks per wave
  constexpr int BR = BM < 32 ? BM : 32;       // rows of one block that are stored
  constexpr int CPR = SB / 16;              // 16-byte chunks per stage row
  constexpr int RPI = 1024 / SB;            // rows per load instruction
  constexpr int KST = SB / 2;               // K values per stage
  constexpr int NSTEP = SB / 32;            // 16-K MFMA steps per stage
  constexpr int KSTEP = NSTEP / KS;         // of which each wave of a block takes
  constexpr int A_BYTES = BM * SB, B_BYTES = BN * SB;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_DMA = A_BYTES / 1024, B_DMA = B_BYTES / 1024;
  static_assert(B_DMA % NW == 0, "B stages split evenly over the waves");
  // A instruction ins goes to wave ins % NW; waves below A_DMA % NW issue
  // one more A load per stage than the others
  constexpr int A_MAX = (A_DMA + NW - 1) / NW, A_MIN = A_DMA / NW, B_PER = B_DMA / NW;
  constexpr int NDMA_MAX = A_MAX + B_PER, NDMA_MIN = A_MIN + B_PER;
  static_assert(NST >= 2 && (NST - 2) * NDMA_MAX <= 63, "stage loads in flight fit the counter");
  constexpr int RING = NST * STAGE;
  static_assert(RING <= 160 * 1024, "LDS");
  constexpr int OPF = 32 * 4 + 16;          // per-wave fp32 strip pitch
  constexpr int OPG = BN * 4 + 16;          // block-wide fp32 strip pitch (SiLU(gate) * up)
  constexpr int PART = KS > 1 ? NCB * FM * 4096 : 0;  // second waves' partial sums
  static_assert(NCB * 32 * OPF <= STAGE && 32 * OPG <= STAGE && PART <= STAGE,
                "staged strips, and before them the partial sums, fit one stage buffer");

  __shared__ __attribute__((aligned(1024))) uint4 smem[RING / 16];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 31, lgrp = lane >> 5;
  const int M = p.M, N = p.N, K = p.K;
  const int64_t lda = p.lda, ldb = p.ldb;
  const int nss = (K + KST - 1) / KST;      // stages
  const int nfull = K / KST;                // stages wholly inside K
  const int glu = p.glu_half;
  const int gshift = glu ? glu - BN / 2 : 0;

  auto swz = [](int r) { return SB >= 256 ? (r & 15) : ((r >> 1) & 7); };
  // Load sources (bytes): instruction ins of a stage covers rows RPI ins ..;
  // lane l fills position l % CPR of row RPI ins + l / CPR, i.e. fetches chunk
  // (l % CPR) ^ swz(row) of that row's SB bytes.
  const int a_cnt = (wave < A_DMA % NW) ? A_MAX : A_MIN;
  uint32_t voA[A_MAX > 0 ? A_MAX : 1], voB[B_PER];
#pragma unroll
  for (int t = 0; t < A_MAX; ++t) {
    const int r = RPI * (wave + NW * t) + lane / CPR;
    voA[t] = (uint32_t)(r * lda * 2) + (uint32_t)(((lane % CPR) ^ swz(r)) << 4);
  }
#pragma unroll
  for (int t = 0; t < B_PER; ++t) {
    const int r = RPI * (wave + NW * t) + lane / CPR;
    const int col = r + (r >= BN / 2 ? gshift : 0);
    voB[t] = (uint32_t)(col * ldb * 2) + (uint32_t)(((lane % CPR) ^ swz(r)) << 4);
  }
  const uint32_t ldsw = __builtin_amdgcn_readfirstlane(lds0 + 1024 * wave);

  // Wave w works on column block cb = w % NCB and, with two waves per block,
  // on MFMA steps kh * KSTEP .. of every stage (kh = w / NCB).
  const int cb = wave % NCB, kh = wave / NCB;
  // Operand reads: A row 32 i + lrow of block i (rows >= BM give zeros), B
  // row 32 cb + lrow; MFMA step t of a stage takes chunk 2 t + lgrp.
  const int ar = lrow & (BR - 1);
  const int br = 32 * cb + lrow;
  const bool a_live = lrow < BM;
  const uint32_t rA = lds0 + (uint32_t)(ar * SB), rB = lds0 + A_BYTES + (uint32_t)(br * SB);
  const int swa = swz(ar), swb = swz(br);

  // A tile's panels (the rows of A and the columns of B it reads) and their
  // valid extents in bytes, to the operand's last element.
  struct Panels {
    const char* a;
    int64_t a_bytes;
    const char* b;
    int64_t b_bytes;
  };
  auto panels_of = [&](int wg_it) -> Panels {
    int wg = wg_it;
    if constexpr (DEBUG) {
      if ((p.flags & kDbgCollide) && wg == 1) wg = 0;  // negative control only
    }
    int32_t tm, tn;
    tile_of(p.map, wg, tm, tn);
    const int m0 = tm * BM, n0 = tn * (glu ? BN / 2 : BN);
    return Panels{reinterpret_cast<const char*>(p.A + (int64_t)m0 * lda),
                  K > 0 ? (((int64_t)(M - 1) * lda + K) - (int64_t)m0 * lda) * 2 : 0,
                  reinterpret_cast<const char*>(p.B + (int64_t)n0 * ldb),
                  K > 0 ? (((int64_t)(N - 1) * ldb + K) - (int64_t)n0 * ldb) * 2 : 0};
  };
  // Stage s of the tile with panels pn into buffer `buf`.
  auto issue_stage = [&](const Panels& pn, int s, int buf) {
    const uint32_t st = (uint32_t)buf * STAGE;
    const i32x4 rsA = make_rsrc(pn.a + (int64_t)s * SB, pn.a_bytes - (int64_t)s * SB);
    const i32x4 rsB = make_rsrc(pn.b + (int64_t)s * SB, pn.b_bytes - (int64_t)s * SB);
#pragma unroll
    for (int t = 0; t < A_MAX; ++t)
      if (t < A_MIN || t < a_cnt) dma16(ldsw + st + 1024 * NW * t, rsA, voA[t], 0u);
#pragma unroll
    for (int t = 0; t < B_PER; ++t) dma16(ldsw + st + A_BYTES + 1024 * NW * t, rsB, voB[t], 0u);
  };

  const int n_tiles = p.map.tiles_m * p.map.tiles_n;
  int gbase = 0;  // buffer of this tile's stage 0
  int pre = 0;    // this tile's leading stages already issued by the previous tile
  for (int wg_it = blockIdx.x; wg_it < n_tiles; wg_it += gridDim.x) {
    int32_t tm, tn;
    {
      int wg = wg_it;
      if constexpr (DEBUG) {
        if ((p.flags & kDbgCollide) && wg == 1) wg = 0;
      }
      tile_of(p.map, wg, tm, tn);
    }
    const int m0 = tm * BM, n0 = tn * (glu ? BN / 2 : BN);
    const Panels cur = panels_of(wg_it);
    // the workgroup's next tile takes its first NST - 1 stages from this
    // tile's last steps (when this tile has that many)
    const bool cross = wg_it + (int)gridDim.x < n_tiles && nss >= NST - 1;
    const Panels nxt = cross ? panels_of(wg_it + gridDim.x) : cur;

    // Wait until this wave's loads of stage s have landed, `after` stages
    // having been issued after it.
    auto wait_after = [&](int after) {
      static_for<0, NST - 1>([&](auto a_c) {
        constexpr int a = decltype(a_c)::value;
        if (after == a) {
          if (NDMA_MAX != NDMA_MIN && a_cnt == A_MAX) wait_vmcnt<a * NDMA_MAX>();
          else wait_vmcnt<a * NDMA_MIN>();
        }
      });
    };

    floatx16 acc[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) acc[i] = floatx16{};
    for (int s = pre; s < NST - 1 && s < nss; ++s) issue_stage(cur, s, (gbase + s) % NST);
    for (int s = 0; s < nss; ++s) {
      // stages issued after s: this tile's, then (cross) the next tile's
      wait_after(cross ? NST - 2 : (nss - 1 < s + NST - 2 ? nss - 1 : s + NST - 2) - s);
      wait_lgkmcnt0();
      block_barrier();
      const int sn = s + NST - 1;
      if (sn < nss) issue_stage(cur, sn, (gbase + sn) % NST);
      else if (cross) issue_stage(nxt, sn - nss, (gbase + sn) % NST);
      const uint32_t so = (uint32_t)((gbase + s) % NST) * STAGE;
      auto step = [&](auto t_c, bool tail) {
        const int t = kh * KSTEP + decltype(t_c)::value;
        const int c = 2 * t + lgrp;
        const int valid = K - (s * KST + 8 * c);  // values of this chunk inside K
        bf16x8 b = lds_read16(rB + so + (uint32_t)((c ^ swb) << 4));
        if (tail) b = keep_first(b, valid);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          bf16x8 a = lds_read16(rA + so + (uint32_t)(32 * i * SB + ((c ^ swa) << 4)));
          if (!a_live) a = bf16x8{};
          if (tail) a = keep_first(a, valid);
          acc[i] = mma(a, b, acc[i]);
        }
      };
      if (s < nfull) {
        static_for<0, KSTEP>([&](auto t_c) { step(t_c, false); });
      } else {
        static_for<0, KSTEP>([&](auto t_c) {
          if (s * KST + 16 * (kh * KSTEP + decltype(t_c)::value) < K) step(t_c, true);
        });
      }
    }

    // Store: the finished accumulators are staged as fp32 in the free ring
    // and written once per element (bias and activation applied there). With
    // two waves per block the second passes its partial sums through LDS
    // (the top of the ring) and the first adds them, always in that order.
    wait_lgkmcnt0();
    block_barrier();
    // the buffer of this tile's last stage: read by now, and the one buffer no
    // load of the next tile is filling
    const uint32_t ebuf = lds0 + (uint32_t)(((gbase + nss + NST - 1) % NST) * STAGE);
    if constexpr (KS > 1) {
      const uint32_t pb = ebuf;
      if (kh == 1) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            lds_store_f4(pb + (uint32_t)((cb * FM + i) * 4096 + q * 1024 + lane * 16),
                         floatx4{acc[i][4 * q], acc[i][4 * q + 1], acc[i][4 * q + 2], acc[i][4 * q + 3]});
      }
      wait_lgkmcnt0();
      block_barrier();
      if (kh == 0) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const floatx4 v = lds_load_f4(pb + (uint32_t)((cb * FM + i) * 4096 + q * 1024 + lane * 16));
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][4 * q + e] += v[e];
          }
      }
      // the strips below reuse the partial sums' bytes
      wait_lgkmcnt0();
      block_barrier();
    }
    if (glu) {
      const EpiOut eo{p.C, p.ldc, M, glu, p.bias, p.act, p.counts, p.flags};
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if (kh == 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            lds_store_f4(ebuf + (uint32_t)(lrow * OPG + (32 * cb + 8 * q + 4 * lgrp) * 4),
                         floatx4{acc[i][4 * q], acc[i][4 * q + 1], acc[i][4 * q + 2], acc[i][4 * q + 3]});
        }
        wait_lgkmcnt0();
        block_barrier();
        store_staged_glu<OUT_BF16, DEBUG>(ebuf, OPG, BR, BN / 2, BR, 0, m0 + 32 * i, n0, tid, NT, eo);
        wait_lgkmcnt0();
        block_barrier();
      }
    } else if (kh == 0) {
      const uint32_t stf = ebuf + (uint32_t)(cb * 32 * OPF);
      const EpiOut eo{p.C, p.ldc, M, N, p.bias, p.act, p.counts, p.flags};
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          lds_store_f4(stf + (uint32_t)(lrow * OPF + (8 * q + 4 * lgrp) * 4),
                       floatx4{acc[i][4 * q], acc[i][4 * q + 1], acc[i][4 * q + 2], acc[i][4 * q + 3]});
        wait_lgkmcnt0();
        store_staged_fused<OUT_BF16, DEBUG>(stf, OPF, BR, 32, m0 + 32 * i, n0 + 32 * cb, lane, 64,
                                            eo);
        wait_lgkmcnt0();
      }
    }
    wait_lgkmcnt0();
    block_barrier();
    gbase = (gbase + nss) % NST;
    pre = cross ? NST - 1 : 0;
  }
}

}  // namespace tg
