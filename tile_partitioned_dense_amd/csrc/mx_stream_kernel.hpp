// mx_stream_kernel.hpp -- MXFP8 / MXFP4 product for few-row outputs (decode
// shapes), where the time is the stream of B's bytes from HBM.
//
// Same operands, formats, ownership and store as mx_kernel.hpp (the OCP MX
// reading of the TorchInductor page's MXFP8 and FP4 GEMMs: E4M3 or E2M1
// elements, one E8M0 scale per 32 along K; B given as its N x K transpose).
// Every BM x BN tile of C (BM = 16, 32 or 64 rows, so one tile row covers a
// decode batch) is owned by one workgroup, which reads A and B as shared
// immutable views and writes its tile once; a persistent grid walks tiles
// wg, wg + grid, ...
//
// What differs from the tile kernel is the K step. A stage is SB = 128 or
// 256 bytes of K per row (two or four of the tile kernel's 64-byte slabs), so
// each direct buffer -> LDS load instruction (one KiB per wave) covers eight
// or four B rows with whole 128-byte lines, instead of sixteen rows with half
// a line each: HBM sees long runs of each weight row. In LDS a stage row is
// SB / 16 16-byte chunks, chunk c of row r at position c ^ swz(r) (swz(r) =
// r & 15 for rows of 256 bytes or more, (r >> 1) & 7 for 128-byte rows), so the sixteen
// rows one MFMA operand read touches (same chunk, consecutive rows) land in
// sixteen distinct bank groups. The loads place the chunks by permuting which
// chunk each lane fetches; every instruction still reads one KiB of whole
// row pieces.
//
// KS waves (one or two) work on each 32-column block of the tile, all its
// rows: wave w takes block w % (BN / 32) and, of every stage's slabs, the
// share (w / (BN / 32)) * SPS / KS ..; every wave issues a share of the
// loads. A wave holds one 32 x 32 accumulator block per 32 rows, transposed
// (as in the tile kernels: the B fragment is the instruction's first operand,
// read once for all blocks); with KS = 2 the second wave of a block adds its
// partial sums into the first's after the K loop, always in that order, and
// the first stores. With BM = 16 the lanes of
// rows 16..31 give zero A operands, so the block's upper half stays zero and
// is never stored. The operand layout, the scale placement (lane r + 32 b
// holds the scale of block b of row r) and the per-format instruction count
// per 64-byte slab are those of mx_kernel.hpp.
//
// Scales: 16 bytes of each row's scale row (eight E4M3 slabs or four E2M1
// slabs: one or more stages, or part of one) are loaded into a ring of LDS
// windows just before the first stage they cover, so the wait that covers
// that stage covers them. A window is stored dword-major (dword d of row r
// at 4 (d R + r), R rows per part), by 4-byte direct loads, so the 32 rows
// one scale read covers sit in 32 consecutive banks.
//
// Each step waits for stage s, passes one barrier (after which every wave is
// done with stage s - 1), loads stage s + NST - 1 into stage s - 1's buffer
// and then runs stage s's MFMAs; NST - 1 stages stay in flight. Each wave
// accumulates its share of K in ascending order in fp32 and the two shares
// of a block meet in a fixed order, so results are bit-identical run to run.
// K must be a multiple of the slab (64 E4M3 or 128 E2M1 values); a
// last stage that is only partly inside K runs only its valid slabs (the
// bytes loaded past a row's end belong to the next row or read as zero and
// are never used).
#pragma once

#include "mx_kernel.hpp"

namespace tg {

template <int BM, int BN, int SB, int NST, int KS, int FMT, bool OUT_BF16, bool DEBUG>
__global__ __launch_bounds__(BN / 32 * KS * 64, 1) void mx_stream_kernel(MxArgs p) {
  static_assert(BM == 16 || BM == 32 || BM == 64, "half a 32-row block, or one or two blocks");
  static_assert(BN % 64 == 0 && BN <= 256, "whole scale-window loads for B");
  static_assert(SB == 128 || SB == 256 || SB == 512, "stage rows of whole 128-byte lines");
  static_assert(FMT == kMxE4M3 || FMT == kMxE2M1, "E4M3 or E2M1 elements");
  static_assert(KS == 1 || KS == 2, "one or two waves per 32-column block");
  constexpr int NCB = BN / 32;               // 32-column blocks
  constexpr int NW = NCB * KS;               // waves (all of them issue loads)
  constexpr int FM = BM < 32 ? 1 : BM / 32;   // 32-row accumulator blocks per wave
  constexpr int BR = BM < 32 ? BM : 32;       // rows of one block that are stored
  constexpr bool FP4 = FMT == kMxE2M1;
  constexpr int HW = FP4 ? 4 : 0;
  constexpr int CPR = SB / 16;              // 16-byte chunks per stage row
  constexpr int RPI = 1024 / SB;            // rows per load instruction
  constexpr int SPS = SB / 64;              // 64-byte slabs per stage
  constexpr int KSL = SPS / KS;             // of which each wave of a block takes
  static_assert(KSL % 2 == 0 || KS == 1, "each wave's slabs start at an even slab");
  constexpr int KPS = FP4 ? 128 : 64;       // K values per slab
  constexpr int SPW = FP4 ? 4 : 8;          // slabs per 16-byte scale window
  constexpr int SSW = SPS < SPW ? SPW / SPS : 1;  // stages per scale window
  constexpr int WPS = SPS > SPW ? SPS / SPW : 1;  // scale windows per stage
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
  constexpr int SWA = 64 * 16;              // window: 64 A-row slots, then the BN B rows,
  constexpr int SWIN = SWA + BN * 16;       // each part dword-major
  // Window v is loaded with the first stage that reads it. With SSW stages
  // per window: stage SSW v, issued in step SSW v - (NST - 1); its buffer
  // takes window v + NWB, issued in step SSW (v + NWB) - (NST - 1), which
  // must come after step SSW (v + 1) - 1, the last to read window v. With WPS
  // windows per stage: windows WPS s .. WPS s + WPS - 1 go with stage s, and
  // window v + WPS NST is issued in step v / WPS + 1, after the only step
  // that reads window v.
  constexpr int NWB = WPS > 1 ? WPS * NST : 1 + (NST - 1 + SSW - 1) / SSW;
  static_assert(WPS > 1 || SSW * (NWB - 1) >= NST - 1,
                "a scale window is reloaded only after its last use");
  constexpr int NWIN = 4 * (1 + BN / 64);   // window load instructions (256 bytes each)
  static_assert(RING + NWB * SWIN <= 160 * 1024, "LDS");

  __shared__ __attribute__((aligned(1024))) uint4 smem[(RING + NWB * SWIN) / 16];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const uint32_t swin0 = lds0 + RING;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 31, lgrp = lane >> 5;
  const int M = p.M, N = p.N, K = p.K;
  const int64_t lda = p.lda, ldb = p.ldb;
  const int nk = K / KPS;                   // 64-byte slabs in a row
  const int nss = (nk + SPS - 1) / SPS;     // stages
  const int kbytes = FP4 ? K / 2 : K;

  auto swz = [](int r) { return SB >= 256 ? (r & 15) : ((r >> 1) & 7); };
  // Load sources: instruction ins of a stage covers rows RPI ins ..; lane l
  // fills position l % CPR of row RPI ins + l / CPR, i.e. fetches chunk
  // (l % CPR) ^ swz(row) of that row's SB bytes.
  const int a_cnt = (wave < A_DMA % NW) ? A_MAX : A_MIN;
  uint32_t voA[A_MAX > 0 ? A_MAX : 1], voB[B_PER];
#pragma unroll
  for (int t = 0; t < A_MAX; ++t) {
    const int r = RPI * (wave + NW * t) + lane / CPR;
    voA[t] = (uint32_t)(r * lda) + (uint32_t)(((lane % CPR) ^ swz(r)) << 4);
  }
#pragma unroll
  for (int t = 0; t < B_PER; ++t) {
    const int r = RPI * (wave + NW * t) + lane / CPR;
    voB[t] = (uint32_t)(r * ldb) + (uint32_t)(((lane % CPR) ^ swz(r)) << 4);
  }
  const uint32_t ldsw = __builtin_amdgcn_readfirstlane(lds0 + 1024 * wave);

  // Wave w works on column block cb = w % NCB and, with two waves per block,
  // on slabs kh * KSL .. of every stage (kh = w / NCB).
  const int cb = wave % NCB, kh = wave / NCB;
  // Operand reads: A row 32 i + lrow of block i (rows >= BM give zeros), B
  // row 32 cb + lrow; slab j of a stage is chunks 4 j + lgrp and 4 j + 2 + lgrp.
  const int ar = lrow & (BR - 1);
  const int br = 32 * cb + lrow;
  const bool a_live = lrow < BM;
  const uint32_t rA = lds0 + (uint32_t)(ar * SB), rB = lds0 + A_BYTES + (uint32_t)(br * SB);
  const int swa = swz(ar), swb = swz(br);
  const int sh = 8 * lgrp;

  const int n_tiles = p.map.tiles_m * p.map.tiles_n;
  for (int wg_it = blockIdx.x; wg_it < n_tiles; wg_it += gridDim.x) {
    int wg = wg_it;
    if constexpr (DEBUG) {
      if ((p.flags & kDbgCollide) && wg == 1) wg = 0;  // negative control only
    }
    int32_t tm, tn;
    tile_of(p.map, wg, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const char* a_panel = reinterpret_cast<const char*>(p.A + (int64_t)m0 * lda);
    const int64_t a_bytes = K > 0 ? ((int64_t)(M - 1) * lda + kbytes) - (int64_t)m0 * lda : 0;
    const char* b_panel = reinterpret_cast<const char*>(p.B + (int64_t)n0 * ldb);
    const int64_t b_bytes = K > 0 ? ((int64_t)(N - 1) * ldb + kbytes) - (int64_t)n0 * ldb : 0;
    const i32x4 rsSA = make_rsrc(p.sA, (int64_t)M * p.ls);
    const i32x4 rsSB = make_rsrc(p.sB, (int64_t)N * p.ls);

    // Window v into buffer v % NWB: instruction u < 4 takes dword u of A
    // scale rows m0 .. m0 + 63 (rows past M read as zero; only the first BM
    // are used), instruction 4 + d (BN / 64) + q dword d of B scale rows
    // n0 + 64 q ..; lane l fetches row (first row) + l.
    auto issue_window = [&](int v) {
      const uint32_t dst = swin0 + (uint32_t)((v % NWB) * SWIN);
#pragma unroll
      for (int u = 0; u < NWIN; ++u) {
        if (u % NW == wave) {
          if (u < 4) {
            dma4(dst + 256 * u, rsSA, (uint32_t)(m0 + lane) * (uint32_t)p.ls + 16u * v + 4u * u, 0u);
          } else {
            const int d = (u - 4) / (BN / 64), q = (u - 4) % (BN / 64);
            dma4(dst + SWA + d * (BN * 4) + 256 * q, rsSB,
                 (uint32_t)(n0 + 64 * q + lane) * (uint32_t)p.ls + 16u * v + 4u * d, 0u);
          }
        }
      }
    };
    auto issue_stage = [&](int s) {
      if constexpr (WPS > 1) {
        for (int w = 0; w < WPS; ++w) issue_window(s * WPS + w);
      } else {
        if (s % SSW == 0) issue_window(s / SSW);
      }
      const uint32_t st = (uint32_t)(s % NST) * STAGE;
      const i32x4 rsA = make_rsrc(a_panel + (int64_t)s * SB, a_bytes - (int64_t)s * SB);
      const i32x4 rsB = make_rsrc(b_panel + (int64_t)s * SB, b_bytes - (int64_t)s * SB);
#pragma unroll
      for (int t = 0; t < A_MAX; ++t)
        if (t < A_MIN || t < a_cnt) dma16(ldsw + st + 1024 * NW * t, rsA, voA[t], 0u);
#pragma unroll
      for (int t = 0; t < B_PER; ++t) dma16(ldsw + st + A_BYTES + 1024 * NW * t, rsB, voB[t], 0u);
    };
    // Wait until this wave's loads of stage s have landed, `after` stages
    // having been issued after it (scale windows among the later loads only
    // make the wait longer).
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
    for (int s = 0; s < NST - 1 && s < nss; ++s) issue_stage(s);
    for (int s = 0; s < nss; ++s) {
      wait_after((nss - 1 < s + NST - 2 ? nss - 1 : s + NST - 2) - s);
      wait_lgkmcnt0();
      block_barrier();
      if (s + NST - 1 < nss) issue_stage(s + NST - 1);
      const uint32_t so = (uint32_t)(s % NST) * STAGE;
      // slab j = kh KSL + jj of the stage; jj and j have the same parity
      auto slab = [&](auto jj_c) {
        constexpr int jj = decltype(jj_c)::value;
        const int j = kh * KSL + jj;
        {
          const int c0 = 4 * j + lgrp, c1 = 4 * j + 2 + lgrp;
          uint4 x = __builtin_bit_cast(uint4, lds_read16(rB + so + (uint32_t)(((c0 ^ swb)) << 4)));
          uint4 y = __builtin_bit_cast(uint4, lds_read16(rB + so + (uint32_t)(((c1 ^ swb)) << 4)));
          const i32x8 bf = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w,
                                 (int)y.x, (int)y.y, (int)y.z, (int)y.w};
          // the scale dword of slab g = SPS s + j: window g / SPW, slab g % SPW
          // of it; E4M3 holds two slabs per dword, E2M1 one
          const int g = SPS * s + j;
          const uint32_t wb = swin0 + (uint32_t)(((g / SPW) % NWB) * SWIN);
          const int sw = g % SPW;
          const int dw = FP4 ? sw : sw / 2;
          const uint32_t vb = *(const __attribute__((address_space(3))) uint32_t*)(uintptr_t)(
              wb + (uint32_t)(SWA + dw * (BN * 4) + br * 4));
          const int sb = (int)(vb >> sh);
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const uint32_t ra = rA + so + (uint32_t)(32 * i * SB);
            x = __builtin_bit_cast(uint4, lds_read16(ra + (uint32_t)(((c0 ^ swa)) << 4)));
            y = __builtin_bit_cast(uint4, lds_read16(ra + (uint32_t)(((c1 ^ swa)) << 4)));
            if (!a_live) x = y = make_uint4(0, 0, 0, 0);
            const i32x8 af = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w,
                                   (int)y.x, (int)y.y, (int)y.z, (int)y.w};
            const uint32_t va = *(const __attribute__((address_space(3))) uint32_t*)(uintptr_t)(
                wb + (uint32_t)(dw * 256 + (32 * i + ar) * 4));
            const int sa = (int)(va >> sh);
            if constexpr (FP4) {
              acc[i] = mma_mx<0, HW>(fp4_half<0>(af), fp4_half<0>(bf), sa, sb, acc[i]);
              acc[i] = mma_mx<2, HW>(fp4_half<1>(af), fp4_half<1>(bf), sa, sb, acc[i]);
            } else {
              acc[i] = mma_mx<2 * (jj % 2), HW>(af, bf, sa, sb, acc[i]);
            }
          }
        }
      };
      if (SPS * (s + 1) <= nk) {
        static_for<0, KSL>(slab);
      } else {
        static_for<0, KSL>([&](auto jj_c) {
          if (SPS * s + kh * KSL + decltype(jj_c)::value < nk) slab(jj_c);
        });
      }
    }

    // Store: the first wave of each block stages its 32 columns (32 rows at a
    // time) as fp32 in the free ring and writes them once per element (with
    // the fused epilogue when asked); with two waves per block the second
    // passes its partial sums through the top of the ring first and the first
    // adds them, always in that order.
    wait_lgkmcnt0();
    block_barrier();
    constexpr int PART = KS > 1 ? NCB * FM * 4096 : 0;
    if constexpr (KS > 1) {
      const uint32_t pb = lds0 + (uint32_t)(RING - PART);
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
    }
    if (kh == 0) {
      constexpr int OPF = 32 * 4 + 16;
      static_assert(NCB * 32 * OPF + PART <= RING, "fp32 strips and partial sums fit the ring");
      const uint32_t stf = lds0 + (uint32_t)(cb * 32 * OPF);
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
  }
}

}  // namespace tg
