// tile64_kernel.hpp -- the 16x16x32-MFMA tile kernel with 64-deep K slabs.
//
// Ownership, the fragment layout, the MFMA and the epilogue are those of
// tile16_kernel.hpp; what differs is the staging. A slab is 64 values of K:
// a K-contiguous operand row (A, column-major B) is 128 bytes in LDS, so each
// direct-to-LDS load instruction moves eight whole 128-byte lines (eight
// lanes per row) instead of sixteen half lines. Measured on gfx950, the
// texture path's work per load instruction, not the bytes moved, was the
// larger part of what the loads cost the 32-deep kernel.
//
// LDS holds two slabs (64 KiB each for 256 x 256 tiles). Per wave and slab s,
// the FM x FN blocks of its sub-tile are taken in 2 * NSTEP phases, one per
// (32-wide k half h, pair of A block rows q):
//   phases before the last: their blocks, reading the next phase's two A
//     fragments (and, at the end of the first k half, the second half's B
//     fragments, each right after the last MFMA that uses the first half's);
//     the loads of slab s + 1 that were not issued yet go out during the
//     first phase, spread over its MFMAs, into the stage slab s - 1 freed;
//   wait for every load of slab s + 1, barrier;
//   last phase: its blocks, reading the next slab's first A fragments and
//     its first-half B fragments, and issuing the first loads of slab s + 2
//     into the stage this slab is leaving.
// A 16-byte chunk c (of 8) of slab row r sits at position c ^ ((r >> 1) & 7)
// of its row: the fragment reads (16 rows, four chunks) measured
// conflict-free with it.
#pragma once

#include "tile16_kernel.hpp"

namespace tg {

__device__ __forceinline__ int swz64(int r) { return (r >> 1) & 7; }

template <int BM, int BN, int WM, int WN, bool BCOL, bool OUT_BF16, bool DEBUG>
__global__ __launch_bounds__(WM * WN * 64, 1) void tile64_gemm_kernel(TileArgs p) {
  constexpr int NW = WM * WN;
  constexpr int NT = NW * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int FQ = 2;             // A blocks (16-row) per phase
  constexpr int NSTEP = FM / FQ;    // phases per k half
  constexpr int NPH = 2 * NSTEP;    // phases per slab
  constexpr int NM = FQ * FN;       // MFMAs per phase
  constexpr int RB = BCOL ? 1 : 2;  // LDS instructions per B fragment
  static_assert(WTM % (16 * FQ) == 0 && WTN % 16 == 0, "wave tile: whole phases of 16-row blocks");
  static_assert(NW == 4 || NW == 8, "one or two waves per SIMD");
  constexpr bool TIED = NW == 4;  // accumulators tied in place (see mma16)
  // one wave per SIMD (no other wave fills the MFMA pipe while this one waits):
  // the steady loop takes its end barrier TL phases before a slab's end and
  // reads every fragment TL phases ahead; a slab's B loads go out in the
  // second k half two slabs ahead, T1 quarters of its A loads after that
  // slab's end barrier and the rest spread over the next slab's first DW
  // phases
  constexpr int TL = 1, DW = 3, T1 = 2;
  static_assert(!TIED || (TL >= 1 && TL <= NSTEP && TL <= 3 && DW < NPH - TL && T1 >= 1 && T1 <= 4),
                "tied schedule");
  constexpr int BK = 64;
  constexpr int A_BYTES = BM * BK * 2;  // per stage
  constexpr int B_BYTES = BN * BK * 2;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_DMA = A_BYTES / 1024;  // one KiB per wave instruction
  constexpr int B_DMA = B_BYTES / 1024;
  static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "slabs are whole KiB");
  static_assert(A_DMA % NW == 0, "A slab splits evenly over the waves");
  constexpr int A_PER = A_DMA / NW;
  constexpr int B_MAX = (B_DMA + NW - 1) / NW;
  constexpr int B_MIN = B_DMA / NW;
  constexpr int PITCH = BN * 2;  // row-major B: bytes per k row
  constexpr int CPR = BN / 8;  // row-major B: 16-byte chunks per k row
  static_assert(A_BYTES <= 65536 - 16 * 1024 && B_BYTES <= 65536, "ds_read immediates within a stage");

  __shared__ __attribute__((aligned(1024))) uint4 smem[2 * STAGE / 16];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave - (wave / WN) * WN;
  const int l16 = lane & 15, lg = lane >> 4;
  const int tG = lane >> 4, tj = (lane >> 2) & 3, tq = lane & 3;

  const int n_tiles = p.map.tiles_m * p.map.tiles_n;
  for (int wg_it = blockIdx.x; wg_it < n_tiles; wg_it += gridDim.x) {
    int wg = wg_it;
    if constexpr (DEBUG) {
      if ((p.flags & kDbgCollide) && wg == 1) wg = 0;  // negative control only
    }
    int32_t tm, tn;
    tile_of(p.map, wg, tm, tn);
    // (see tile16_kernel.hpp: the K loop keeps only its own waits)
    if constexpr (TIED) wait_vmcnt<0>();
    const int M = p.M, N = p.N, K = p.K;
    const int64_t lda = p.lda, ldb = p.ldb;
    const int glu = p.glu_half;
    const int gshift = glu ? glu - BN / 2 : 0;
    const int m0 = tm * BM, n0 = tn * (glu ? BN / 2 : BN);

    const char* a_panel = reinterpret_cast<const char*>(p.A + (int64_t)m0 * lda);
    const int64_t a_bytes = K > 0 ? (((int64_t)(M - 1) * lda + K) - (int64_t)m0 * lda) * 2 : 0;
    const char* b_panel = reinterpret_cast<const char*>(BCOL ? p.B + (int64_t)n0 * ldb : p.B + n0);
    const int64_t b_bytes = K <= 0 ? 0
                            : BCOL ? (((int64_t)(N - 1) * ldb + K) - (int64_t)n0 * ldb) * 2
                                   : (((int64_t)(K - 1) * ldb + N) - n0) * 2;
    const int64_t a_step = BK * 2;
    const int64_t b_step = BCOL ? BK * 2 : BK * ldb * 2;

    // ---- per-lane DMA source offsets (bytes): eight lanes per 128-byte row
    uint32_t voA[A_PER];
#pragma unroll
    for (int t = 0; t < A_PER; ++t) {
      const int ins = wave + NW * t;
      const int r = 8 * ins + (lane >> 3);
      const int c = (lane & 7) ^ swz64(r);
      voA[t] = (uint32_t)(r * lda * 2) + c * 16;
    }
    const int b_cnt = (wave < B_DMA % NW) ? B_MAX : B_MIN;
    uint32_t voB[B_MAX];
#pragma unroll
    for (int t = 0; t < B_MAX; ++t) {
      const int ins = wave + NW * t;
      if constexpr (BCOL) {
        const int r = 8 * ins + (lane >> 3);
        const int c = (lane & 7) ^ swz64(r);
        voB[t] = (uint32_t)((r + (r >= BN / 2 ? gshift : 0)) * ldb * 2) + c * 16;
      } else {
        const int q = 64 * ins + lane;
        const int row = q / CPR, pc = q - (q / CPR) * CPR;
        const int lc = swzB<CPR>(pc, row);
        voB[t] = (uint32_t)(row * ldb * 2) + lc * 16 + (lc >= CPR / 2 ? 2 * gshift : 0);
      }
    }

    const int nk = (K + BK - 1) / BK;
    // Slabs loaded by DMA; the rest (a K tail, and with a row-major B and an
    // odd N the slab holding B's last value, whose dword straddles the end of
    // the resource and would read as zero) go through registers.
    const int nk_full = (!BCOL && (N & 1)) ? (K - 1) / BK : K / BK;

    // Whole slab s into stage s & 1 (DMA, or the register path past nk_full).
    auto issue_slab = [&](int s) {
      const int st = s & 1;
      const uint32_t la = lds0 + st * STAGE;
      const uint32_t lb = la + A_BYTES;
      if (s < nk_full) {
        const i32x4 rsA = make_rsrc(a_panel + s * a_step, a_bytes - s * a_step);
        const i32x4 rsB = make_rsrc(b_panel + s * b_step, b_bytes - s * b_step);
#pragma unroll
        for (int t = 0; t < A_PER; ++t) dma16(la + 1024 * (wave + NW * t), rsA, voA[t], 0u);
#pragma unroll
        for (int t = 0; t < B_MAX; ++t)
          if (t < B_MIN || t < b_cnt) dma16(lb + 1024 * (wave + NW * t), rsB, voB[t], 0u);
      } else {
        const int k0 = s * BK;
        uint4* dA = reinterpret_cast<uint4*>(reinterpret_cast<char*>(smem) + st * STAGE);
        uint4* dB = reinterpret_cast<uint4*>(reinterpret_cast<char*>(smem) + st * STAGE + A_BYTES);
        for (int q = tid; q < BM * 8; q += NT) {
          const int r = q >> 3, c = q & 7;
          const uint4 v = (m0 + r < M) ? load8_masked(p.A + (int64_t)(m0 + r) * lda, k0 + 8 * c, K)
                                       : make_uint4(0, 0, 0, 0);
          dA[r * 8 + (c ^ swz64(r))] = v;
        }
        if constexpr (BCOL) {
          for (int q = tid; q < BN * 8; q += NT) {
            const int r = q >> 3, c = q & 7;
            const int col = n0 + r + (r >= BN / 2 ? gshift : 0);
            const uint4 v = (col < N) ? load8_masked(p.B + (int64_t)col * ldb, k0 + 8 * c, K)
                                      : make_uint4(0, 0, 0, 0);
            dB[r * 8 + (c ^ swz64(r))] = v;
          }
        } else {
          for (int q = tid; q < BK * CPR; q += NT) {
            const int row = q / CPR, pc = q - (q / CPR) * CPR;
            const int lc = swzB<CPR>(pc, row);
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
    // DMA units [lo, hi) of full slab s (units 0 .. A_PER-1: this wave's A
    // loads, then its b_cnt B loads).
    // (one wave per SIMD: its b_cnt B loads first, then its A loads)
    auto issue_units = [&](int s, int lo, int hi) {
      const uint32_t la = lds0 + (s & 1) * STAGE;
      const uint32_t lb = la + A_BYTES;
      const i32x4 rsA = make_rsrc(a_panel + s * a_step, a_bytes - s * a_step);
      const i32x4 rsB = make_rsrc(b_panel + s * b_step, b_bytes - s * b_step);
      if constexpr (TIED) {
#pragma unroll
        for (int t = 0; t < B_MAX; ++t)
          if (t < b_cnt && t >= lo && t < hi) dma16(lb + 1024 * (wave + NW * t), rsB, voB[t], 0u);
#pragma unroll
        for (int t = 0; t < A_PER; ++t)
          if (b_cnt + t >= lo && b_cnt + t < hi) dma16(la + 1024 * (wave + NW * t), rsA, voA[t], 0u);
      } else {
#pragma unroll
        for (int t = 0; t < A_PER; ++t)
          if (t >= lo && t < hi) dma16(la + 1024 * (wave + NW * t), rsA, voA[t], 0u);
#pragma unroll
        for (int t = 0; t < B_MAX; ++t)
          if (t < b_cnt && A_PER + t >= lo && A_PER + t < hi)
            dma16(lb + 1024 * (wave + NW * t), rsB, voB[t], 0u);
      }
    };

    floatx4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{};

    // ---- LDS read addresses: one lane base per stage and k half (stage
    // offsets exceed a ds_read immediate); block offsets are immediates.
    uint32_t rA[2][2], rB[2][2];  // [stage][k half]
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t ch = (uint32_t)(((4 * h + lg) ^ swz64(l16)) << 4);
        rA[st][h] = lds0 + st * STAGE + (uint32_t)((wm * WTM + l16) * 128) + ch;
        rB[st][h] = lds0 + st * STAGE + A_BYTES + (uint32_t)((wn * WTN + l16) * 128) + ch;
      }
    uint32_t rT[BCOL ? 1 : FN][2];  // row-major B: per block and stage
#pragma unroll
    for (int j = 0; j < (BCOL ? 1 : FN); ++j) {
      const int n = wn * WTN + 16 * j + 4 * tq;
      const int col = (swzB<CPR>(n >> 3, 8 * tG + tj) << 3) | (n & 7);
#pragma unroll
      for (int st = 0; st < 2; ++st)
        rT[j][st] = lds0 + st * STAGE + A_BYTES + (uint32_t)((8 * tG + tj) * PITCH + col * 2);
    }

    bf16x8 aS[2][FQ];  // A fragments: phase p uses set p & 1 while set (p + 1) & 1 is read
    bf16x8 bq[FN];     // B fragments of the current k half

    // A block I, k half H of the slab in stage ST (run-time ST, H allowed)
    auto readA = [&](int st, int h, int i) -> bf16x8 {
      return lds_read16(rA[st][h] + (uint32_t)(i * 2048));
    };
    auto readB = [&](int st, int h, int j) -> bf16x8 {
      if constexpr (BCOL) {
        return lds_read16(rB[st][h] + (uint32_t)(j * 2048));
      } else {
        const uint32_t b = rT[j][st] + (uint32_t)(h * 32 * PITCH);
        const i16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(uintptr_t)(b));
        const i16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(uintptr_t)(b + 4 * PITCH));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };

    // Order of a phase's MFMAs: the last phase of a k half goes column by
    // column (so B fragment j of the next half can be read right after the
    // last MFMA using this half's), the others row by row.
    auto blk = [](int q, int k) constexpr {
      return q == NSTEP - 1 ? (k % FQ) * FN + (k / FQ) : k;  // i * FN + j within the phase
    };
    auto nreads = [](int q, int k) constexpr {
      if (q != NSTEP - 1) return (k * FQ) % NM == 0 ? 1 : 0;
      return (k < FQ ? 1 : 0) + (k % FQ == FQ - 1 ? RB : 0);
    };

    // Steady loop: slab s + 1 full and s + 2 full, so every load is a DMA.
    const bool steady_on = nk_full >= 3;
    constexpr int NDMA_MAX = A_PER + B_MAX;
    const int ndma = A_PER + b_cnt;
    // units issued after a slab's barrier for slab + 2
    constexpr int NA1 = (A_PER * T1 + 3) / 4;  // one wave per SIMD: A loads after the end barrier
    const int nh1 = TIED ? b_cnt + NA1 : (ndma + 1) / 2;

    // ---- prologue
    if (nk > 0) {
      issue_slab(0);
      if (steady_on) {
        issue_units(1, 0, nh1);
        // slab 0 has landed once at most slab 1's nh1 loads remain
        constexpr int NMAX = A_PER + B_MAX, NMIN = A_PER + B_MIN;
        if (B_MAX != B_MIN && b_cnt == B_MAX)
          wait_vmcnt<TIED ? B_MAX + NA1 : (NMAX + 1) / 2>();
        else
          wait_vmcnt<TIED ? B_MIN + NA1 : (NMIN + 1) / 2>();
      } else {
        wait_vmcnt<0>();
      }
      block_barrier();
#pragma unroll
      for (int f = 0; f < FQ; ++f) aS[0][f] = readA(0, 0, f);
#pragma unroll
      for (int j = 0; j < FN; ++j) bq[j] = readB(0, 0, j);
    }

    const uint32_t ldsw = __builtin_amdgcn_readfirstlane(lds0 + 1024 * wave);
    auto steady = [&](auto bc_c) -> int {
      constexpr int BC = decltype(bc_c)::value;
      constexpr int NDMA = A_PER + BC;
      constexpr int NH1 = (NDMA + 1) / 2;  // of slab s + 2, in slab s's last phase
      constexpr int NH2 = NDMA - NH1;      // of slab s + 1, in slab s's first phase
      auto dma_first = [](int t, int n) constexpr { return ((2 * t + 1) * NM) / (2 * n); };
      auto dma_last = [](int t, int n) constexpr { return ((2 * t + 1) * NM) / (2 * n); };
      int s = 0;
      if (!steady_on) return 0;
      auto unit = [&](auto stg_c, auto u_c, const i32x4& rA_, const i32x4& rB_) {
        constexpr int STG = decltype(stg_c)::value, U = decltype(u_c)::value;
        if constexpr (U < A_PER)
          dma16_off<STG * STAGE + 1024 * NW * U>(ldsw, rA_, voA[U]);
        else
          dma16_off<STG * STAGE + A_BYTES + 1024 * NW * (U - A_PER)>(ldsw, rB_, voB[U - A_PER]);
      };
      i32x4 rsA1 = make_rsrc(a_panel + 1 * a_step, a_bytes - 1 * a_step);  // slab s + 1
      i32x4 rsB1 = make_rsrc(b_panel + 1 * b_step, b_bytes - 1 * b_step);
      i32x4 rsA2 = make_rsrc(a_panel + 2 * a_step, a_bytes - 2 * a_step);  // slab s + 2
      i32x4 rsB2 = make_rsrc(b_panel + 2 * b_step, b_bytes - 2 * b_step);
      // pairs of slabs, so the stage of each is a compile-time constant
      for (; s + 4 <= nk_full; s += 2) {
        static_for<0, 2>([&](auto st_c) {
          constexpr int ST = decltype(st_c)::value;  // stage of this slab
          static_for<0, NPH>([&](auto p_c) {
            constexpr int P = decltype(p_c)::value;
            constexpr int H = P / NSTEP, Q = P % NSTEP;
            constexpr bool LAST = P == NPH - 1;
            if constexpr (LAST) {
              // every load of slab + 1 has landed; this wave's reads of this
              // slab have returned (the last phase's A fragments were read in
              // the phase before), so after the barrier no wave reads this
              // slab's stage any more and slab + 2 may fill it
              wait_vmcnt<0>();
              wait_lgkmcnt0();
              block_barrier();
            }
            static_for<0, NM>([&](auto k_c) {
              constexpr int k = decltype(k_c)::value;
              constexpr int b = blk(Q, k), i = b / FN, j = b % FN;
              mma16<false>(acc[Q * FQ + i][j], aS[P & 1][i], bq[j]);
              if constexpr (Q != NSTEP - 1) {
                // next phase's A fragments, same k half
                if constexpr ((k * FQ) % NM == 0)
                  aS[(P + 1) & 1][k * FQ / NM] = readA(ST, H, (Q + 1) * FQ + k * FQ / NM);
              } else if constexpr (!LAST) {
                // end of the first k half: the second half's first A fragments
                // and its B fragments
                if constexpr (k < FQ) aS[(P + 1) & 1][k] = readA(ST, 1, k);
                if constexpr (k % FQ == FQ - 1) bq[j] = readB(ST, 1, j);
              } else {
                // last phase: the next slab's
                if constexpr (k < FQ) aS[0][k] = readA(ST ^ 1, 0, k);
                if constexpr (k % FQ == FQ - 1) bq[j] = readB(ST ^ 1, 0, j);
              }
              if constexpr (H == 0) {
                static_for<0, NH2>([&](auto t_c) {
                  constexpr int t = decltype(t_c)::value;
                  if constexpr (dma_first(t, NH2) == Q * NM + k)
                    unit(std::integral_constant<int, ST ^ 1>{}, std::integral_constant<int, NH1 + t>{}, rsA1, rsB1);
                });
              }
              if constexpr (LAST) {
                static_for<0, NH1>([&](auto t_c) {
                  constexpr int t = decltype(t_c)::value;
                  if constexpr (dma_last(t, NH1) == k)
                    unit(std::integral_constant<int, ST>{}, std::integral_constant<int, t>{}, rsA2, rsB2);
                });
              }
            });
            static_for<0, NM>([&](auto k_c) {
              constexpr int k = decltype(k_c)::value;
              constexpr int nr = nreads(Q, k);
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);
            });
          });
          advance_rsrc(rsA1, (uint32_t)a_step);
          advance_rsrc(rsB1, (uint32_t)b_step);
          advance_rsrc(rsA2, (uint32_t)a_step);
          advance_rsrc(rsB2, (uint32_t)b_step);
        });
      }
      return s;
    };
    // The steady loop of the one-wave-per-SIMD tiles (the same slabs, stages
    // and loads, the same ownership; a different order):
    //   phase P of slab s (P = 0 .. NPH-1): its FQ x FN blocks column by
    //     column, reading the A fragments of the phase TL later (a ring of four
    //     phase sets), in phases NSTEP-TL .. NSTEP-1 the second k half's B
    //     fragments (B has one register set per k half), and from the barrier
    //     on the next slab's first-half B fragments;
    //   before phase NSTEP (the second k half): barrier, after which no wave
    //     reads slab s's B any more (its second-half fragments were read in
    //     the phases before), so slab s + 2's B loads go out, spread over
    //     phases NSTEP .. NPH-TL-1;
    //   before phase NPH-TL: wait for every load of slab s + 1, barrier (no
    //     wave reads slab s's stage any more: its last fragments were read
    //     TL phases ahead); then slab s + 2's first NA1 A loads, the rest
    //     spread over slab s + 1's first DW phases.
    auto steady_tied = [&](auto bc_c) -> int {
      constexpr int BC = decltype(bc_c)::value;
      constexpr int NA2 = A_PER - NA1;          // A loads of slab s + 1 in slab s's first DW phases
      constexpr int PB = NPH - TL;              // the end barrier comes before phase PB
      constexpr int BW = PB - NSTEP;            // phases the B loads spread over
      static_assert(BW >= 1 && DW <= NSTEP, "tied load windows");
      constexpr int NBR = FN / TL;              // B reads per phase (the last phase takes the rest)
      if (!steady_on) return 0;
      auto unit = [&](auto stg_c, auto u_c, const i32x4& rA_, const i32x4& rB_) {
        constexpr int STG = decltype(stg_c)::value, U = decltype(u_c)::value;
        if constexpr (U < A_PER)
          dma16_off<STG * STAGE + 1024 * NW * U>(ldsw, rA_, voA[U]);
        else
          dma16_off<STG * STAGE + A_BYTES + 1024 * NW * (U - A_PER)>(ldsw, rB_, voB[U - A_PER]);
      };
      bf16x8 aR[4][FQ];  // A fragments of phase g in set g % 4
      bf16x8 bR[2][FN];  // B fragments of k half h
      // slab 0: the A fragments of its first TL phases, its first-half B
      static_for<0, TL>([&](auto p_c) {
        constexpr int P = decltype(p_c)::value;
        static_for<0, FQ>([&](auto f_c) {
          constexpr int F = decltype(f_c)::value;
          aR[P][F] = readA(0, P / NSTEP, (P % NSTEP) * FQ + F);
        });
      });
      static_for<0, FN>([&](auto j_c) {
        constexpr int J = decltype(j_c)::value;
        bR[0][J] = readB(0, 0, J);
      });
      i32x4 rsA1 = make_rsrc(a_panel + 1 * a_step, a_bytes - 1 * a_step);  // slab s + 1
      i32x4 rsB1 = make_rsrc(b_panel + 1 * b_step, b_bytes - 1 * b_step);
      i32x4 rsA2 = make_rsrc(a_panel + 2 * a_step, a_bytes - 2 * a_step);  // slab s + 2
      i32x4 rsB2 = make_rsrc(b_panel + 2 * b_step, b_bytes - 2 * b_step);
      int s = 0;
      for (; s + 4 <= nk_full; s += 2) {
        tied_entry();
        static_for<0, 2>([&](auto st_c) {
          constexpr int ST = decltype(st_c)::value;  // stage of this slab
          static_for<0, NPH>([&](auto p_c) {
            constexpr int P = decltype(p_c)::value;
            constexpr int G = ST * NPH + P;  // phase within the two slabs
            constexpr int H = P / NSTEP, Q = P % NSTEP;
            if constexpr (P == NSTEP) {
              wait_lgkmcnt0();
              block_barrier();
            }
            if constexpr (P == PB) {
              wait_vmcnt<BC>();  // all but slab s + 2's B loads
              wait_lgkmcnt0();
              block_barrier();
            }
            // this phase's reads, in order: A of phase P + TL, then its B share
            constexpr int PA = P + TL;  // phase whose A fragments are read
            constexpr bool B1 = P >= NSTEP - TL && P < NSTEP;  // second half's B
            constexpr bool B0 = P >= PB;                       // next slab's first-half B
            constexpr int BI = B1 ? P - (NSTEP - TL) : B0 ? P - PB : 0;
            constexpr int BLO = BI * NBR, BHI = (BI == TL - 1) ? FN : BLO + NBR;
            constexpr int NRD = FQ + ((B1 || B0) ? BHI - BLO : 0);
            static_for<0, NM>([&](auto k_c) {
              constexpr int k = decltype(k_c)::value;
              constexpr int i = k % FQ, j = k / FQ;
              mma16<true>(acc[Q * FQ + i][j], aR[G % 4][i], bR[H][j]);
              static_for<0, NRD>([&](auto r_c) {
                constexpr int r = decltype(r_c)::value;
                if constexpr (((2 * r + 1) * NM) / (2 * NRD) == k) {
                  if constexpr (r < FQ) {
                    if constexpr (PA < NPH)
                      aR[(G + TL) % 4][r] = readA(ST, PA / NSTEP, (PA % NSTEP) * FQ + r);
                    else
                      aR[(G + TL) % 4][r] = readA(ST ^ 1, (PA - NPH) / NSTEP, ((PA - NPH) % NSTEP) * FQ + r);
                  } else if constexpr (B1) {
                    bR[1][BLO + r - FQ] = readB(ST, 1, BLO + r - FQ);
                  } else {
                    bR[0][BLO + r - FQ] = readB(ST ^ 1, 0, BLO + r - FQ);
                  }
                }
              });
              if constexpr (P < DW) {  // A of slab s + 1, the rest
                static_for<0, NA2>([&](auto t_c) {
                  constexpr int t = decltype(t_c)::value;
                  if constexpr (((2 * t + 1) * DW * NM) / (2 * NA2) == P * NM + k)
                    unit(std::integral_constant<int, ST ^ 1>{}, std::integral_constant<int, NA1 + t>{}, rsA1, rsB1);
                });
              }
              if constexpr (P >= NSTEP && P < PB) {  // B of slab s + 2
                static_for<0, BC>([&](auto t_c) {
                  constexpr int t = decltype(t_c)::value;
                  if constexpr (((2 * t + 1) * BW * NM) / (2 * BC) == (P - NSTEP) * NM + k)
                    unit(std::integral_constant<int, ST>{}, std::integral_constant<int, A_PER + t>{}, rsA2, rsB2);
                });
              }
              if constexpr (P >= PB) {  // A of slab s + 2, the first NA1
                static_for<0, NA1>([&](auto t_c) {
                  constexpr int t = decltype(t_c)::value;
                  if constexpr (((2 * t + 1) * TL * NM) / (2 * NA1) == (P - PB) * NM + k)
                    unit(std::integral_constant<int, ST>{}, std::integral_constant<int, t>{}, rsA2, rsB2);
                });
              }
            });
          });
          advance_rsrc(rsA1, (uint32_t)a_step);
          advance_rsrc(rsB1, (uint32_t)b_step);
          advance_rsrc(rsA2, (uint32_t)a_step);
          advance_rsrc(rsB2, (uint32_t)b_step);
        });
      }
      return s;
    };
    int s0 = 0;
    if constexpr (TIED) {
      if constexpr (B_MAX != B_MIN) {
        if (b_cnt == B_MAX) s0 = steady_tied(std::integral_constant<int, B_MAX>{});
        else s0 = steady_tied(std::integral_constant<int, B_MIN>{});
      } else {
        s0 = steady_tied(std::integral_constant<int, B_MIN>{});
      }
    } else if constexpr (B_MAX != B_MIN) {
      if (b_cnt == B_MAX) s0 = steady(std::integral_constant<int, B_MAX>{});
      else s0 = steady(std::integral_constant<int, B_MIN>{});
    } else {
      s0 = steady(std::integral_constant<int, B_MIN>{});
    }
    (void)NDMA_MAX;

    // ---- remaining slabs: slab s0 has landed (the last barrier, or the
    // prologue), and when the steady loop ran, the first nh1 loads of slab
    // s0 + 1 are in flight. Complete slab s0 + 1, then one slab at a time:
    // compute it, wait for the next, barrier, load the one after.
    if (nk > 0 && s0 + 1 < nk) {
      if (steady_on && s0 + 1 < nk_full) issue_units(s0 + 1, nh1, ndma);
      else issue_slab(s0 + 1);
    }
    for (int s = s0; s < nk; ++s) {
      if constexpr (TIED) tied_entry();
      const int st = s & 1;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int q = 0; q < NSTEP; ++q) {
#pragma unroll
          for (int f = 0; f < FQ; ++f) aS[0][f] = readA(st, h, q * FQ + f);
          if (q == 0) {
#pragma unroll
            for (int j = 0; j < FN; ++j) bq[j] = readB(st, h, j);
          }
#pragma unroll
          for (int i = 0; i < FQ; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) mma16<TIED>(acc[q * FQ + i][j], aS[0][i], bq[j]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<0>();   // slab s + 1 (if any) has landed
      wait_lgkmcnt0();   // this wave's reads of slab s have returned
      block_barrier();   // every wave is done with slab s's stage
      if (s + 2 < nk) issue_slab(s + 2);
    }

    // ---- epilogue (as in tile16_kernel.hpp): 16-row strips staged in the
    // now idle stages, stored as 16-byte row chunks, each element once
    if constexpr (TIED) settle_tied();
    constexpr int ESZ = OUT_BF16 ? 2 : 4;
    constexpr int RING = 2 * STAGE;
    constexpr int SH = 16;
    constexpr int OPITCH = WTN * ESZ + 16;
    static_assert(NW * SH * OPITCH <= RING, "a staged strip of every wave fits the stages");
    constexpr int CH = WTN * ESZ / 16;
    constexpr int EPC = 16 / ESZ;
    __syncthreads();
    if (glu) {
      constexpr int OPG = BN * 4 + 16;
      static_assert(WM * SH * OPG <= RING, "a block-wide fp32 strip fits the stages");
      static_assert(BN / 2 % 8 == 0 && BN / 2 / 4 <= NT, "whole output chunks per block row");
      const EpiOut eo{p.C, p.ldc, M, glu, p.bias, p.act, p.counts, p.flags};
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (TIED) pin_row(acc[i]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          lds_store_f4(lds0 + (uint32_t)((wm * SH + l16) * OPG + (wn * WTN + 16 * j + 4 * lg) * 4),
                       acc[i][j]);
        __syncthreads();
        store_staged_glu<OUT_BF16, DEBUG>(lds0, OPG, WM * SH, BN / 2, SH, WTM, m0 + 16 * i, n0, tid,
                                          NT, eo);
        __syncthreads();
      }
      continue;
    }
    if (p.bias != nullptr || p.act != kActNone) {
      constexpr int OPF = WTN * 4 + 16;
      static_assert(NW * SH * OPF <= RING, "an fp32 strip of every wave fits the stages");
      static_assert(WTN / 4 <= 64, "one wave covers a staged row in 16-byte chunks");
      const uint32_t stf = lds0 + (uint32_t)(wave * SH * OPF);
      const EpiOut eo{p.C, p.ldc, M, N, p.bias, p.act, p.counts, p.flags};
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (TIED) pin_row(acc[i]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          lds_store_f4(stf + (uint32_t)(l16 * OPF + (16 * j + 4 * lg) * 4), acc[i][j]);
        wait_lgkmcnt0();
        store_staged_fused<OUT_BF16, DEBUG>(stf, OPF, SH, WTN, m0 + wm * WTM + 16 * i, n0 + wn * WTN,
                                            lane, 64, eo);
        wait_lgkmcnt0();
      }
      wait_lgkmcnt0();
      block_barrier();
      continue;
    }
    const uint32_t stg = lds0 + (uint32_t)(wave * SH * OPITCH);
    const bool full_mn = (m0 + BM <= M) && (n0 + BN <= N);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if constexpr (TIED) pin_row(acc[i]);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint32_t a = stg + (uint32_t)(l16 * OPITCH + (16 * j + 4 * lg) * ESZ);
        const floatx4 v = acc[i][j];
        if constexpr (OUT_BF16) {
          const u32x2v w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *(__attribute__((address_space(3))) u32x2v*)(uintptr_t)a = w;
        } else {
          *(__attribute__((address_space(3))) floatx4*)(uintptr_t)a = v;
        }
      }
      wait_lgkmcnt0();
      const int grow0 = m0 + wm * WTM + 16 * i;
      const int gcol0 = n0 + wn * WTN;
#pragma unroll
      for (int c0 = 0; c0 < SH * CH; c0 += 64) {
        const int c = c0 + lane;
        if (SH * CH % 64 != 0 && c >= SH * CH) break;
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
    wait_lgkmcnt0();
    block_barrier();
  }
}

}  // namespace tg
