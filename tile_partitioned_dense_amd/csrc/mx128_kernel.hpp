// mx128_kernel.hpp -- the MX tile kernel (mx_kernel.hpp) with 128-byte stage
// rows: two MX slabs per stage, so each direct-to-LDS load instruction moves
// eight whole 128-byte lines instead of sixteen half lines.
//
// What it keeps from mx_kernel.hpp: the operands and scales (MxArgs), the
// ownership and tile walk, v_mfma_scale_f32_32x32x64_f8f6f4 per 32 x 32 block
// and slab with the B fragment as the first operand, the scale windows (16
// bytes of every tile row, loaded straight into LDS with the stage that holds
// their first slab, row r shifted by (r / 8) % 4 dwords), the per-slab take of
// the scales into the register set of the slab's parity, fp32 accumulation in
// ascending K and the staged store. Measured with the counters on the MLP
// shard, the 64-byte form sent 2.3 times the L2 requests per byte of the bf16
// kernels and stalled its texture unit five times as often per load.
//
// What differs is the staging and its schedule, which are those of the tied
// one-wave-per-SIMD bf16 kernel (tile64_kernel.hpp, steady_tied): two stages
// of (BM + BN) x 128 bytes; stage S holds slabs 2 S (bytes 0-63 of each row)
// and 2 S + 1 (bytes 64-127), 16-byte chunk q of row r at position q ^ (r % 8)
// (a fragment read, eight consecutive rows of one chunk per pass, then touches
// eight different bank groups). A stage is taken in eight phases, one per
// (slab half h, 32-row block i): the phase's MFMAs over the wave's column
// blocks (both E2M1 halves of a chunk in turn), with the next phase's A
// fragment read one phase ahead; B fragments are held per slab. A barrier at
// the start of the stage's second slab frees its B rows (the second slab's B
// fragments were read in the phase before), so the B loads two stages ahead
// spread over phases 4-6; a barrier before the last phase, after a wait for
// the next stage's loads, frees the A rows, and half of the A loads two stages
// ahead follow it, the rest spread over the next stage's first three phases
// together with the scale window that stage starts.
#pragma once

#include "mx_kernel.hpp"
#include "tile16_kernel.hpp"

namespace tg {

// One scaled 32 x 32 x 64 step of a C block held transposed (as mma_mx), its
// accumulator tied in place and the instruction kept where the loop puts it.
// The compiler does not see an MFMA in it: the two wait states a vector write
// of an operand (the scale shifts) needs before it are issued here (2 of the
// instruction's 64 cycles), and settle_tied() waits out its result latency.
// E4M3 operands are 8 registers (32 elements), E2M1 operands 4 (32 four-bit
// elements: one 16-byte chunk, half of a staged fragment).
template <int OPSEL>
__device__ __forceinline__ void mma_mx_tied(floatx16& acc, const i32x8& a_frag, const i32x8& b_frag,
                                            int a_scale, int b_scale) {
  static_assert(OPSEL == 0 || OPSEL == 2, "scale bytes used here");
  if constexpr (OPSEL == 0)
    asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
                 : "+a"(acc) : "v"(b_frag), "v"(a_frag), "v"(b_scale), "v"(a_scale));
  else
    asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[1,1,0]"
                 : "+a"(acc) : "v"(b_frag), "v"(a_frag), "v"(b_scale), "v"(a_scale));
}
template <int OPSEL>
__device__ __forceinline__ void mma_mx_tied(floatx16& acc, const i32x4& a_half, const i32x4& b_half,
                                            int a_scale, int b_scale) {
  static_assert(OPSEL == 0 || OPSEL == 2, "scale bytes used here");
  if constexpr (OPSEL == 0)
    asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
                 : "+a"(acc) : "v"(b_half), "v"(a_half), "v"(b_scale), "v"(a_scale));
  else
    asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[1,1,0] cbsz:4 blgp:4"
                 : "+a"(acc) : "v"(b_half), "v"(a_half), "v"(b_scale), "v"(a_scale));
}
template <int H>
__device__ __forceinline__ i32x4 fp4_part(const i32x8& f) {
  return i32x4{f[4 * H], f[4 * H + 1], f[4 * H + 2], f[4 * H + 3]};
}

template <int BM, int BN, int WM, int WN, int FMT, bool OUT_BF16, bool DEBUG>
__global__ __launch_bounds__(WM * WN * 64, 1) void mx128_gemm_kernel(MxArgs p) {
  static_assert(FMT == 0 || FMT == 1, "E4M3 or E2M1 elements");
  constexpr int NW = WM * WN;
  static_assert(NW == 4, "one wave per SIMD");
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  constexpr bool FP4 = FMT == kMxE2M1;
  constexpr int RB = 128;                 // bytes per row and stage (two slabs)
  constexpr int KPS = FP4 ? 128 : 64;     // K elements per slab
  constexpr int SPW = FP4 ? 4 : 8;        // slabs per scale window (16 scale bytes per row)
  constexpr int A_BYTES = BM * RB, B_BYTES = BN * RB;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_DMA = A_BYTES / 1024, B_DMA = B_BYTES / 1024;
  static_assert(A_DMA % NW == 0 && B_DMA % NW == 0, "stages split evenly over the waves");
  constexpr int A_PER = A_DMA / NW, B_PER = B_DMA / NW;
  constexpr int RING = 2 * STAGE;
  constexpr int SWIN = (BM + BN) * 16;    // one scale window: 16 bytes per row
  // Window w (slabs SPW w ..) lives in buffer (w + 1) % NWB and goes out with
  // the A loads that stage SPW w / 2 - 1 spreads over its first phases, after
  // the end barrier of the stage before, which every wave passes only once it
  // has taken the scales of slab SPW w - 3; the last take that reads the
  // buffer it replaces, window w - NWB + 1's, is slab SPW (w - NWB + 1) + T1
  // (as in mx_kernel.hpp).
  constexpr int T1 = FP4 ? 2 : 4;
  constexpr int NWB = 1 + (3 + T1 + SPW - 1) / SPW;
  static_assert(SPW * (NWB - 1) - 3 >= T1, "a scale window is reloaded only after its last use");
  static_assert(SPW % 2 == 0, "a window starts with a stage");
  static_assert(BM % 64 == 0 && BN % 64 == 0, "scale windows are whole KiB per wave instruction");
  constexpr int SA_DMA = BM / 64, SB_DMA = BN / 64;
  static_assert(RING + NWB * SWIN <= 160 * 1024, "LDS");
  // schedule (see the header): phases per stage, the end barrier's phase,
  // the phases the B loads spread over, the A loads after the end barrier and
  // the phases the rest of them spread over
  constexpr int NPH = 2 * FM;             // (slab half, 32-row block)
  constexpr int PMID = FM, PB = NPH - 1;
  constexpr int BW = PB - PMID, DW = 3;
  constexpr int NA1 = A_PER / 2, NA2 = A_PER - NA1;
  static_assert(BW >= 1 && DW < PB, "load windows");
  constexpr int NBLK = FM * FN;
  constexpr int MPP = (FP4 ? 2 : 1) * FN;  // MFMAs per phase

  __shared__ __attribute__((aligned(1024))) uint4 smem[(RING + NWB * SWIN) / 16];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave - (wave / WN) * WN;
  const int lrow = lane & 31, lgrp = lane >> 5;
  const int M = p.M, N = p.N, K = p.K;
  const int64_t lda = p.lda, ldb = p.ldb;
  const int nk = K / KPS;                 // slabs (K is a multiple of KPS)
  const int nst = (nk + 1) / 2;           // stages (the last one half empty when nk is odd)
  const int kbytes = FP4 ? K / 2 : K;     // bytes of K in a row

  // per-lane DMA source offsets within a stage (bytes): eight lanes per row,
  // chunk (lane % 8) ^ (row % 8) of it
  uint32_t voA[A_PER], voB[B_PER];
#pragma unroll
  for (int t = 0; t < A_PER; ++t) {
    const int r = 8 * (wave + NW * t) + (lane >> 3);
    voA[t] = (uint32_t)(r * lda) + (uint32_t)(((lane & 7) ^ (r & 7)) << 4);
  }
#pragma unroll
  for (int t = 0; t < B_PER; ++t) {
    const int r = 8 * (wave + NW * t) + (lane >> 3);
    voB[t] = (uint32_t)(r * ldb) + (uint32_t)(((lane & 7) ^ (r & 7)) << 4);
  }
  const uint32_t ldsw = __builtin_amdgcn_readfirstlane(lds0 + 1024 * wave);
  // fragment read bases: row lrow of the wave's first block, chunk 4 h + lgrp
  // (part 0) and 4 h + 2 + lgrp (part 1) of slab half h
  const int sw = lrow & 7;
  const uint32_t rowA = lds0 + (uint32_t)((wm * WTM + lrow) * RB);
  const uint32_t rowB = lds0 + A_BYTES + (uint32_t)((wn * WTN + lrow) * RB);
  auto chunk = [&](int h, int part) -> uint32_t { return (uint32_t)(((4 * h + 2 * part + lgrp) ^ sw) << 4); };

  const int n_tiles = p.map.tiles_m * p.map.tiles_n;
  for (int wg_it = blockIdx.x; wg_it < n_tiles; wg_it += gridDim.x) {
    int wg = wg_it;
    if constexpr (DEBUG) {
      if ((p.flags & kDbgCollide) && wg == 1) wg = 0;  // negative control only
    }
    int32_t tm, tn;
    tile_of(p.map, wg, tm, tn);
    // (as in tile16_kernel.hpp: settle the previous tile's loads and stores
    // here, not at the K loop's head)
    wait_vmcnt<0>();
    const int m0 = tm * BM, n0 = tn * BN;
    const char* a_panel = reinterpret_cast<const char*>(p.A + (int64_t)m0 * lda);
    const int64_t a_bytes = K > 0 ? ((int64_t)(M - 1) * lda + kbytes) - (int64_t)m0 * lda : 0;
    const char* b_panel = reinterpret_cast<const char*>(p.B + (int64_t)n0 * ldb);
    const int64_t b_bytes = K > 0 ? ((int64_t)(N - 1) * ldb + kbytes) - (int64_t)n0 * ldb : 0;

    const int sh = 8 * lgrp;
    const i32x4 rsSA = make_rsrc(p.sA, (int64_t)M * p.ls);
    const i32x4 rsSB = make_rsrc(p.sB, (int64_t)N * p.ls);
    const uint32_t swin0 = lds0 + RING;
    // window w into buffer (w + 1) % NWB (as in mx_kernel.hpp)
    auto issue_window = [&](int w) {
      const uint32_t dst = swin0 + (uint32_t)(((w + 1) % NWB) * SWIN);
      const int g = (lane >> 3) & 3;
      const int kofs = (w < 0 && g == 0) ? 0 : 16 * w + 4 * g;
      const uint32_t k8 = (uint32_t)kofs;
#pragma unroll
      for (int q = 0; q < SA_DMA; ++q)
        if (q % NW == wave)
          dma16(dst + 1024 * q, rsSA, (uint32_t)(m0 + 64 * q + lane) * (uint32_t)p.ls + k8, 0u);
#pragma unroll
      for (int q = 0; q < SB_DMA; ++q)
        if (q % NW == wave)
          dma16(dst + BM * 16 + 1024 * q, rsSB, (uint32_t)(n0 + 64 * q + lane) * (uint32_t)p.ls + k8, 0u);
    };
    auto rsA_of = [&](int st) { return make_rsrc(a_panel + (int64_t)st * RB, a_bytes - (int64_t)st * RB); };
    auto rsB_of = [&](int st) { return make_rsrc(b_panel + (int64_t)st * RB, b_bytes - (int64_t)st * RB); };
    // a stage's loads in issue order: its B loads (positions 0 .. B_PER - 1),
    // its first NA1 A loads, its scale window if it starts one (position
    // B_PER + NA1), the other A loads; positions [lo, hi) of stage st into
    // buffer st % 2
    auto issue_units = [&](int st, int lo, int hi) {
      const uint32_t la = ldsw + (uint32_t)((st & 1) * STAGE);
      const i32x4 rsA = rsA_of(st), rsB = rsB_of(st);
#pragma unroll
      for (int t = 0; t < B_PER; ++t)
        if (t >= lo && t < hi) dma16(la + A_BYTES + 1024 * NW * t, rsB, voB[t], 0u);
#pragma unroll
      for (int t = 0; t < NA1; ++t)
        if (B_PER + t >= lo && B_PER + t < hi) dma16(la + 1024 * NW * t, rsA, voA[t], 0u);
      if (B_PER + NA1 >= lo && B_PER + NA1 < hi && (2 * st) % SPW == 0) issue_window(2 * st / SPW);
#pragma unroll
      for (int t = NA1; t < A_PER; ++t)
        if (B_PER + t + 1 >= lo && B_PER + t + 1 < hi) dma16(la + 1024 * NW * t, rsA, voA[t], 0u);
    };
    constexpr int NU = A_PER + B_PER;

    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = floatx16{};

    // scales of slab s in set s % 2, shifted per lane (as in mx_kernel.hpp)
    int sca[2][FM], scb[2][FN];
    uint32_t rsa[FM], rsb[FN];
    const uint32_t sra = (uint32_t)((wm * WTM + lrow) * 16);
    const uint32_t srb = (uint32_t)(BM * 16 + (wn * WTN + lrow) * 16);
    auto fetch_scales = [&](int s) {
      const int w = s / SPW;
      const int dw = FP4 ? (s % SPW) : ((s % SPW) >> 1);
      const int g = (lrow >> 3) & 3;
      const int buf = dw < g ? w : w + 1;
      const uint32_t wb = swin0 + (uint32_t)((buf % NWB) * SWIN) + (uint32_t)(4 * ((dw - g) & 3));
      const uint32_t wa = wb + sra, wbb = wb + srb;
#pragma unroll
      for (int i = 0; i < FM; ++i)
        rsa[i] = *(const __attribute__((address_space(3))) uint32_t*)(uintptr_t)(wa + 512u * i);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        rsb[j] = *(const __attribute__((address_space(3))) uint32_t*)(uintptr_t)(wbb + 512u * j);
    };
    auto take_scales = [&](int set) {
#pragma unroll
      for (int i = 0; i < FM; ++i) sca[set][i] = (int)(rsa[i] >> sh);
#pragma unroll
      for (int j = 0; j < FN; ++j) scb[set][j] = (int)(rsb[j] >> sh);
    };
    auto frag = [&](uint32_t row_base, int st, int h, int blk) -> i32x8 {
      const uint32_t b = row_base + (uint32_t)(st * STAGE + blk * 32 * RB);
      const uint4 x = __builtin_bit_cast(uint4, lds_read16(b + chunk(h, 0)));
      const uint4 y = __builtin_bit_cast(uint4, lds_read16(b + chunk(h, 1)));
      return i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
    };
    // the MFMAs of block row i, slab half H (scale set H), with A fragment a
    auto row_mfmas = [&](auto h_c, int i, const i32x8& a, const i32x8 (&bq)[FN], auto k_hook) {
      constexpr int H = decltype(h_c)::value;
      static_for<0, MPP>([&](auto k_c) {
        constexpr int k = decltype(k_c)::value;
        constexpr int j = k % FN;
        if constexpr (FP4) {
          constexpr int m = k / FN;
          mma_mx_tied<2 * m>(acc[i][j], fp4_part<m>(a), fp4_part<m>(bq[j]), sca[H][i], scb[H][j]);
        } else {
          mma_mx_tied<2 * H>(acc[i][j], a, bq[j], sca[H][i], scb[H][j]);
        }
        k_hook(k_c);
        __builtin_amdgcn_sched_barrier(0);
      });
    };

    // ---- prologue: windows -1 and 0, stage 0 whole, stage 1's B loads and
    // first A loads; stage 0 landed, slab 0's scales and first fragments read
    const bool steady_on = nst >= 4;
    const int nh1 = B_PER + NA1;  // positions issued for stage S + 2 within stage S
    if (nk > 0) {
      issue_window(-1);
      issue_units(0, 0, NU + 1);
      if (nst > 1) {
        if (steady_on) {
          issue_units(1, 0, nh1);
          wait_vmcnt<B_PER + NA1>();
        } else {
          issue_units(1, 0, NU + 1);
          wait_vmcnt<NU>();  // (stage 1 starts no window: SPW > 2)
        }
      } else {
        wait_vmcnt<0>();
      }
      block_barrier();
      fetch_scales(0);
    }

    // ---- steady loop: stages S, S + 1 per iteration (their buffers fixed),
    // stages S + 2 and S + 3 loaded meanwhile
    int S = 0;
    if (steady_on) {
      i32x8 aR[2];      // A fragment of phase g in set g % 2
      i32x8 bR[2][FN];  // B fragments of slab half h
      aR[0] = frag(rowA, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < FN; ++j) bR[0][j] = frag(rowB, 0, 0, j);
      for (; S + 4 <= nst; S += 2) {
        static_for<0, 2>([&](auto st_c) {
          constexpr int ST = decltype(st_c)::value;  // buffer of this stage
          const int cur = S + ST;
          const i32x4 rsA1 = rsA_of(cur + 1), rsA2 = rsA_of(cur + 2), rsB2 = rsB_of(cur + 2);
          const uint32_t l1 = ldsw + (uint32_t)((ST ^ 1) * STAGE), l2 = ldsw + (uint32_t)(ST * STAGE);
          static_for<0, NPH>([&](auto p_c) {
            constexpr int P = decltype(p_c)::value;
            constexpr int H = P / FM, I = P % FM;
            if constexpr (P == 0) {
              take_scales(0);
              if constexpr (FP4) fetch_scales(2 * cur + 1);
              if ((2 * (cur + 1)) % SPW == 0) issue_window(2 * (cur + 1) / SPW);
            }
            if constexpr (P == PMID) {
              take_scales(1);
              wait_lgkmcnt0();
              block_barrier();
            }
            if constexpr (P == PB) {
              wait_vmcnt<B_PER>();  // all but stage cur + 2's B loads
              wait_lgkmcnt0();
              block_barrier();
              fetch_scales(2 * cur + 2);
            }
            // reads of this phase: the next phase's A fragment, then (phase
            // PMID - 1) the second slab's B fragments or (phase PB) the next
            // stage's first-slab B fragments
            constexpr bool RB1 = P == PMID - 1, RB0 = P == PB;
            constexpr int NRD = 1 + ((RB1 || RB0) ? FN : 0);
            auto hook = [&](auto k_c) {
              constexpr int k = decltype(k_c)::value;
              static_for<0, NRD>([&](auto r_c) {
                constexpr int r = decltype(r_c)::value;
                if constexpr (((2 * r + 1) * MPP) / (2 * NRD) == k) {
                  if constexpr (r == 0) {
                    if constexpr (P + 1 < NPH)
                      aR[(P + 1) & 1] = frag(rowA, ST, (P + 1) / FM, (P + 1) % FM);
                    else
                      aR[0] = frag(rowA, ST ^ 1, 0, 0);
                  } else if constexpr (RB1) {
                    bR[1][r - 1] = frag(rowB, ST, 1, r - 1);
                  } else {
                    bR[0][r - 1] = frag(rowB, ST ^ 1, 0, r - 1);
                  }
                }
              });
              if constexpr (P < DW) {  // the rest of stage cur + 1's A loads
                static_for<0, NA2>([&](auto t_c) {
                  constexpr int t = decltype(t_c)::value;
                  if constexpr (((2 * t + 1) * DW * MPP) / (2 * NA2) == P * MPP + k)
                    dma16(l1 + 1024 * NW * (NA1 + t), rsA1, voA[NA1 + t], 0u);
                });
              }
              if constexpr (P >= PMID && P < PB) {  // stage cur + 2's B loads
                static_for<0, B_PER>([&](auto t_c) {
                  constexpr int t = decltype(t_c)::value;
                  if constexpr (((2 * t + 1) * BW * MPP) / (2 * B_PER) == (P - PMID) * MPP + k)
                    dma16(l2 + A_BYTES + 1024 * NW * t, rsB2, voB[t], 0u);
                });
              }
              if constexpr (P == PB) {  // stage cur + 2's first A loads
                static_for<0, NA1>([&](auto t_c) {
                  constexpr int t = decltype(t_c)::value;
                  if constexpr (((2 * t + 1) * MPP) / (2 * NA1) == k)
                    dma16(l2 + 1024 * NW * t, rsA2, voA[t], 0u);
                });
              }
            };
            row_mfmas(std::integral_constant<int, H>{}, I, aR[P & 1], bR[H], hook);
          });
        });
      }
    }

    // ---- remaining stages, one at a time: stage S has landed (the last
    // barrier, or the prologue) and its first slab's scales are fetched; with
    // the steady loop, stage S + 1's first nh1 positions are in flight
    if (nk > 0 && S + 1 < nst && steady_on) issue_units(S + 1, nh1, NU + 1);
    for (; S < nst; ++S) {
      const int st = S & 1;
      const bool two = 2 * S + 1 < nk;
      __builtin_amdgcn_sched_barrier(0);
      take_scales(0);
      if (FP4 && two) fetch_scales(2 * S + 1);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        i32x8 bq[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) bq[j] = frag(rowB, st, 0, j);
        row_mfmas(std::integral_constant<int, 0>{}, i, frag(rowA, st, 0, i), bq, [](auto) {});
      }
      if (two) {
        take_scales(1);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          i32x8 bq[FN];
#pragma unroll
          for (int j = 0; j < FN; ++j) bq[j] = frag(rowB, st, 1, j);
          row_mfmas(std::integral_constant<int, 1>{}, i, frag(rowA, st, 1, i), bq, [](auto) {});
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<0>();   // stage S + 1 (if any) has landed
      wait_lgkmcnt0();   // this wave's reads of stage S have returned
      block_barrier();   // every wave is done with stage S's buffer
      if (S + 2 < nst) issue_units(S + 2, 0, NU + 1);
      // (after the last slab: dwords of a buffer in bounds, never used)
      fetch_scales(2 * S + 2);
    }

    // ---- store (as in mx_kernel.hpp): fp32 strips staged in the free ring,
    // each element written once (with the fused epilogue when asked)
    settle_tied();
    __syncthreads();
    {
      constexpr int OPF = WTN * 4 + 16;
      constexpr int SHF = (NW * 32 * OPF <= RING) ? 32 : 16;
      static_assert(NW * SHF * OPF <= RING, "an fp32 strip of every wave fits the ring");
      static_assert(WTN / 4 <= 64, "one wave covers a staged row in 16-byte chunks");
      const uint32_t stf = lds0 + (uint32_t)(wave * SHF * OPF);
      const EpiOut eo{p.C, p.ldc, M, N, p.bias, p.act, p.counts, p.flags};
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) asm volatile("" : "+a"(acc[i][j]));  // (see settle_tied)
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
    }
    wait_lgkmcnt0();
    block_barrier();
  }
}

}  // namespace tg
