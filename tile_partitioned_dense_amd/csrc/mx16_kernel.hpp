// mx16_kernel.hpp -- the MX tile kernel on 16 x 16 x 128 scaled MFMA blocks.
//
// The 32 x 32 x 64 kernels (mx_kernel.hpp, mx128_kernel.hpp) need wave tiles
// of whole 32-column blocks, so a 7168-wide output takes 256 x 256 tiles: 896
// of them, four rounds on 224 of the 256 compute units. Blocks of 16 x 16
// allow 256 x 224 tiles (four waves of 128 x 112): 1024 tiles, four full
// rounds. The operands, scales, ownership, tile walk and output are those of
// mx_kernel.hpp (MxArgs; fp32 accumulation in ascending K; each element
// written once).
//
// v_mfma_scale_f32_16x16x128_f8f6f4 takes 128 values of K per block. Probed on
// the device with a one-wave kernel (integer elements, per-block scales that
// differ along K): lane l holds row l % 16 of its operand; for E4M3 its 32
// bytes are bytes 16 g .. 16 g + 15 and 64 + 16 g .. 64 + 16 g + 15 of the
// 128-byte K step (g = l / 16), for E2M1 its 16 bytes are bytes 16 g ..
// 16 g + 15 of the 64-byte K step; the scale of block b (32 values) of row r
// comes from lane r + 16 b. One scale dword of a row therefore covers one K
// step, and lane l takes its byte l / 16 (shifted down per lane; the
// instruction's byte select stays 0).
//
// Staging: two stages of (BM + BN) x 128 bytes (one E4M3 K step or two E2M1
// ones per row), chunk c of row r at position c ^ ((r >> 1) & 7) as in
// tile64_kernel.hpp, whose fragment reads (16 rows, chunks g and 4 + g)
// these are. A fragment is read as both chunks: one E4M3 operand, or the two
// E2M1 operands of the stage's K steps. Scale windows hold 16 bytes of every
// row (four K steps) and travel with the stage that starts them, as in the
// other MX kernels; 16 rows 16 bytes apart meet 16 different banks, so the
// windows need no offset.
//
// Per wave and stage, one phase per 16-row A block: its FN MFMAs (2 FN for
// E2M1: first K step, then second) over B fragments held in registers for the
// whole stage, the next phase's A fragment read during it. The next stage's B
// fragments are read over the phases from PW on, after a barrier at PW that
// waits for that stage's B loads; every wave is then past the reads of this
// stage's B rows (done in the stage before), so the B loads two stages ahead
// go out over phases PW .. PB - 1 into them. A barrier before the last phase
// waits for the next stage's A loads and frees this stage's A rows (their
// last fragment was read a phase ahead); half of the A loads two stages ahead
// follow it, the rest go out over the next stage's first DW phases with the
// scale window that stage starts.
#pragma once

#include "mx128_kernel.hpp"

namespace tg {

// One scaled 16 x 16 x 128 step of a C block held transposed (lane l: row
// l % 16, columns 4 (l / 16) .. + 3), the accumulator tied in place as in
// mma_mx_tied. E4M3 operands are 8 registers, E2M1 operands 4. Unlike
// mma_mx_tied it issues no wait states of its own (two per instruction cost
// the 16-cycle E2M1 form 5% of its shard): the vector writes its operands
// can follow are the scale shifts, which take_scales() ends with a wait, and
// the accumulators' zeroing, which settle_tied(acc) ends; the hazard check
// of the built code covers the rest.
__device__ __forceinline__ void mma16_mx_tied(floatx4& acc, const i32x8& a_frag, const i32x8& b_frag,
                                              int a_scale, int b_scale) {
  asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+a"(acc) : "v"(b_frag), "v"(a_frag), "v"(b_scale), "v"(a_scale));
}
__device__ __forceinline__ void mma16_mx_tied(floatx4& acc, const i32x4& a_half, const i32x4& b_half,
                                              int a_scale, int b_scale) {
  asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
               : "+a"(acc) : "v"(b_half), "v"(a_half), "v"(b_scale), "v"(a_scale));
}

template <int BM, int BN, int WM, int WN, int FMT, bool OUT_BF16, bool DEBUG>
__global__ __launch_bounds__(WM * WN * 64, 1) void mx16_gemm_kernel(MxArgs p) {
  static_assert(FMT == 0 || FMT == 1, "E4M3 or E2M1 elements");
  constexpr int NW = WM * WN;
  static_assert(NW == 4, "one wave per SIMD");
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  static_assert(WTM % 16 == 0 && WTN % 16 == 0 && BM % 16 == 0 && WTN % 16 == 0,
                "wave tiles of whole 16-row blocks at multiples of 16 rows");
  constexpr bool FP4 = FMT == kMxE2M1;
  constexpr int RB = 128;                 // bytes per row and stage
  constexpr int KH = FP4 ? 2 : 1;         // K steps (128 values each) per stage
  constexpr int SPW = 4;                  // K steps per scale window (16 bytes per row)
  constexpr int A_BYTES = BM * RB, B_BYTES = BN * RB;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_DMA = A_BYTES / 1024, B_DMA = B_BYTES / 1024;
  static_assert(A_DMA % NW == 0 && B_DMA % NW == 0, "stages split evenly over the waves");
  constexpr int A_PER = A_DMA / NW, B_PER = B_DMA / NW;
  constexpr int RING = 2 * STAGE;
  static_assert(BM % 64 == 0, "scale windows of A are whole 64-row loads");
  constexpr int BNP = (BN + 63) / 64 * 64;  // B rows of a window (whole 64-row loads)
  constexpr int SWIN = (BM + BNP) * 16;
  // Window w (K steps SPW w ..) lives in buffer w % 2. It goes out at the
  // first phase of the stage before its first stage; the buffer's previous
  // window, w - 2, was last read (its last K step's scales) at the end of a
  // stage at least two stages earlier, and every wave has passed a barrier
  // since.
  constexpr int NWB = 2;
  constexpr int SA_DMA = BM / 64, SB_DMA = BNP / 64;
  static_assert(RING + NWB * SWIN <= 160 * 1024, "LDS");
  constexpr int NPH = FM;                 // phases per stage: one per 16-row A block
  constexpr int PW = 2, PB = NPH - 1;     // barriers: next stage's B landed / its A landed
  constexpr int BW = PB - PW, DW = 2;
  constexpr int NA1 = A_PER / 2, NA2 = A_PER - NA1;
  static_assert(BW >= 1 && DW <= PW, "load windows (the wait at PW counts the A loads before it)");
  constexpr int MPP = KH * FN;            // MFMAs per phase

  __shared__ __attribute__((aligned(1024))) uint4 smem[(RING + NWB * SWIN) / 16];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave - (wave / WN) * WN;
  const int l16 = lane & 15, lg = lane >> 4;
  const int M = p.M, N = p.N, K = p.K;
  const int64_t lda = p.lda, ldb = p.ldb;
  const int nk = K / 128;                 // K steps (K is a multiple of 128)
  const int nst = (nk + KH - 1) / KH;     // stages (E2M1: the last one half empty when nk is odd)
  const int kbytes = FP4 ? K / 2 : K;     // bytes of K in a row

  // per-lane DMA source offsets within a stage (bytes): eight lanes per row,
  // chunk (lane % 8) ^ ((row >> 1) % 8) of it
  uint32_t voA[A_PER], voB[B_PER];
#pragma unroll
  for (int t = 0; t < A_PER; ++t) {
    const int r = 8 * (wave + NW * t) + (lane >> 3);
    voA[t] = (uint32_t)(r * lda) + (uint32_t)(((lane & 7) ^ ((r >> 1) & 7)) << 4);
  }
#pragma unroll
  for (int t = 0; t < B_PER; ++t) {
    const int r = 8 * (wave + NW * t) + (lane >> 3);
    voB[t] = (uint32_t)(r * ldb) + (uint32_t)(((lane & 7) ^ ((r >> 1) & 7)) << 4);
  }
  const uint32_t ldsw = __builtin_amdgcn_readfirstlane(lds0 + 1024 * wave);
  // fragment reads: row l16 of the wave's first block, chunks lg and 4 + lg
  const int sw = (l16 >> 1) & 7;
  const uint32_t rowA = lds0 + (uint32_t)((wm * WTM + l16) * RB);
  const uint32_t rowB = lds0 + A_BYTES + (uint32_t)((wn * WTN + l16) * RB);
  const uint32_t ch0 = (uint32_t)((lg ^ sw) << 4), ch1 = (uint32_t)(((4 + lg) ^ sw) << 4);
  const int sh = 8 * lg;                  // this lane's scale byte of a K step's dword

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

    const i32x4 rsSA = make_rsrc(p.sA, (int64_t)M * p.ls);
    const i32x4 rsSB = make_rsrc(p.sB, (int64_t)N * p.ls);
    const uint32_t swin0 = lds0 + RING;
    // window w: bytes 16 w .. 16 w + 15 of every row's scales into buffer w % 2
    // (one lane per row; rows past M or N read as zero)
    auto issue_window = [&](int w) {
      const uint32_t dst = swin0 + (uint32_t)((w % NWB) * SWIN);
      const uint32_t k8 = (uint32_t)(16 * w);
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
      if (B_PER + NA1 >= lo && B_PER + NA1 < hi && (KH * st) % SPW == 0) issue_window(KH * st / SPW);
#pragma unroll
      for (int t = NA1; t < A_PER; ++t)
        if (B_PER + t + 1 >= lo && B_PER + t + 1 < hi) dma16(la + 1024 * NW * t, rsA, voA[t], 0u);
    };
    constexpr int NU = A_PER + B_PER;

    floatx4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{};
    settle_tied(acc);  // (the zeroing is a vector write of every MFMA's accumulator)

    // scale dwords of a stage's K steps (raw, then shifted to this lane's byte)
    uint32_t rsa[KH][FM], rsb[KH][FN];
    int sca[KH][FM], scb[KH][FN];
    const uint32_t sra = (uint32_t)((wm * WTM + l16) * 16);
    const uint32_t srb = (uint32_t)(BM * 16 + (wn * WTN + l16) * 16);
    auto fetch_scales = [&](int st) {
#pragma unroll
      for (int h = 0; h < KH; ++h) {
        const int s = KH * st + h;
        const uint32_t wb = swin0 + (uint32_t)(((s / SPW) % NWB) * SWIN) + (uint32_t)(4 * (s % SPW));
#pragma unroll
        for (int i = 0; i < FM; ++i)
          rsa[h][i] = *(const __attribute__((address_space(3))) uint32_t*)(uintptr_t)(wb + sra + 256u * i);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          rsb[h][j] = *(const __attribute__((address_space(3))) uint32_t*)(uintptr_t)(wb + srb + 256u * j);
      }
    };
    auto take_scales = [&]() {
#pragma unroll
      for (int h = 0; h < KH; ++h) {
#pragma unroll
        for (int i = 0; i < FM; ++i) sca[h][i] = (int)(rsa[h][i] >> sh);
#pragma unroll
        for (int j = 0; j < FN; ++j) scb[h][j] = (int)(rsb[h][j] >> sh);
      }
      // every shift before one wait of two states, every MFMA after it
#pragma unroll
      for (int h = 0; h < KH; ++h) {
#pragma unroll
        for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(sca[h][i]));
#pragma unroll
        for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(scb[h][j]));
      }
      asm volatile("s_nop 1");
    };
    auto frag = [&](uint32_t row_base, int st, int blk) -> i32x8 {
      const uint32_t b = row_base + (uint32_t)(st * STAGE + blk * 16 * RB);
      const uint4 x = __builtin_bit_cast(uint4, lds_read16(b + ch0));
      const uint4 y = __builtin_bit_cast(uint4, lds_read16(b + ch1));
      return i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
    };
    // MFMA k of block row i's phase (E2M1: K step k / FN), A fragment a
    auto one_mfma = [&](auto k_c, int i, const i32x8& a, const i32x8 (&bq)[FN]) {
      constexpr int k = decltype(k_c)::value;
      constexpr int h = k / FN, j = k % FN;
      if constexpr (FP4)
        mma16_mx_tied(acc[i][j], fp4_part<h>(a), fp4_part<h>(bq[j]), sca[h][i], scb[h][j]);
      else
        mma16_mx_tied(acc[i][j], a, bq[j], sca[0][i], scb[0][j]);
    };

    // ---- prologue: stage 0 whole (with window 0), stage 1's B loads and
    // first A loads; stage 0 landed, its scales fetched
    const bool steady_on = nst >= 4;
    const int nh1 = B_PER + NA1;  // positions issued for stage S + 2 within stage S
    if (nk > 0) {
      issue_units(0, 0, NU + 1);
      if (nst > 1) {
        if (steady_on) {
          issue_units(1, 0, nh1);
          wait_vmcnt<B_PER + NA1>();
        } else {
          issue_units(1, 0, NU + 1);
          wait_vmcnt<NU>();  // (stage 1 starts no window: SPW > KH)
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
      i32x8 aR[2];      // A fragment of phase P in set P % 2
      i32x8 bR[2][FN];  // B fragments of the stage in buffer b
      aR[0] = frag(rowA, 0, 0);
#pragma unroll
      for (int j = 0; j < FN; ++j) bR[0][j] = frag(rowB, 0, j);
      for (; S + 4 <= nst; S += 2) {
        static_for<0, 2>([&](auto st_c) {
          constexpr int ST = decltype(st_c)::value;  // buffer of this stage
          const int cur = S + ST;
          const i32x4 rsA1 = rsA_of(cur + 1), rsA2 = rsA_of(cur + 2), rsB2 = rsB_of(cur + 2);
          const uint32_t l1 = ldsw + (uint32_t)((ST ^ 1) * STAGE), l2 = ldsw + (uint32_t)(ST * STAGE);
          static_for<0, NPH>([&](auto p_c) {
            constexpr int P = decltype(p_c)::value;
            if constexpr (P == 0) {
              take_scales();
              if ((KH * (cur + 1)) % SPW == 0) issue_window(KH * (cur + 1) / SPW);
            }
            if constexpr (P == PW) {
              wait_vmcnt<A_PER>();  // stage cur + 1's B loads (its A loads came after them)
              wait_lgkmcnt0();
              block_barrier();
            }
            if constexpr (P == PB) {
              wait_vmcnt<B_PER>();  // all but stage cur + 2's B loads
              wait_lgkmcnt0();
              block_barrier();
              fetch_scales(cur + 1);
            }
            // reads of this phase: the next phase's A fragment (the next
            // stage's first in the last phase), then from PW on the next
            // stage's B fragments assigned to this phase
            constexpr int JLO = P < PW ? FN : ((P - PW) * FN + (NPH - PW) - 1) / (NPH - PW);
            constexpr int JHI = P < PW ? FN : ((P - PW + 1) * FN + (NPH - PW) - 1) / (NPH - PW);
            constexpr int NRD = 1 + (JHI - JLO);
            auto hook = [&](auto k_c) {
              constexpr int k = decltype(k_c)::value;
              static_for<0, NRD>([&](auto r_c) {
                constexpr int r = decltype(r_c)::value;
                if constexpr (((2 * r + 1) * MPP) / (2 * NRD) == k) {
                  if constexpr (r == 0) {
                    if constexpr (P + 1 < NPH)
                      aR[(P + 1) & 1] = frag(rowA, ST, P + 1);
                    else
                      aR[0] = frag(rowA, ST ^ 1, 0);
                  } else {
                    bR[ST ^ 1][JLO + r - 1] = frag(rowB, ST ^ 1, JLO + r - 1);
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
              if constexpr (P >= PW && P < PB) {  // stage cur + 2's B loads
                static_for<0, B_PER>([&](auto t_c) {
                  constexpr int t = decltype(t_c)::value;
                  if constexpr (((2 * t + 1) * BW * MPP) / (2 * B_PER) == (P - PW) * MPP + k)
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
            static_for<0, MPP>([&](auto k_c) {
              one_mfma(k_c, P, aR[P & 1], bR[ST]);
              hook(k_c);
              __builtin_amdgcn_sched_barrier(0);
            });
          });
        });
      }
    }

    // ---- remaining stages, one at a time: stage S has landed (the last
    // barrier, or the prologue) and its scales are fetched; with the steady
    // loop, stage S + 1's first nh1 positions are in flight
    if (nk > 0 && S + 1 < nst && steady_on) issue_units(S + 1, nh1, NU + 1);
    for (; S < nst; ++S) {
      const int st = S & 1;
      const bool two = KH * S + 1 < nk;  // (E2M1) the stage's second K step exists
      __builtin_amdgcn_sched_barrier(0);
      take_scales();
      i32x8 bq[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) bq[j] = frag(rowB, st, j);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const i32x8 a = frag(rowA, st, i);
        static_for<0, FN>([&](auto k_c) { one_mfma(k_c, i, a, bq); });
        if constexpr (FP4) {
          if (two)
            static_for<0, FN>([&](auto k_c) {
              one_mfma(std::integral_constant<int, FN + decltype(k_c)::value>{}, i, a, bq);
            });
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<0>();   // stage S + 1 (if any) has landed
      wait_lgkmcnt0();   // this wave's reads of stage S have returned
      block_barrier();   // every wave is done with stage S's buffer
      if (S + 2 < nst) issue_units(S + 2, 0, NU + 1);
      // (after the last stage: dwords of a window buffer, in bounds, unused)
      fetch_scales(S + 1);
    }

    // ---- store (as in tile64_kernel.hpp's fused path): fp32 strips of 16
    // rows staged in the free ring, each element written once (with the fused
    // epilogue when asked)
    settle_tied();
    __syncthreads();
    {
      constexpr int SH = 16;
      constexpr int OPF = WTN * 4 + 16;
      static_assert(NW * SH * OPF <= RING, "an fp32 strip of every wave fits the ring");
      static_assert(WTN / 4 <= 64, "one wave covers a staged row in 16-byte chunks");
      const uint32_t stf = lds0 + (uint32_t)(wave * SH * OPF);
      const EpiOut eo{p.C, p.ldc, M, N, p.bias, p.act, p.counts, p.flags};
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        pin_row(acc[i]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          lds_store_f4(stf + (uint32_t)(l16 * OPF + (16 * j + 4 * lg) * 4), acc[i][j]);
        wait_lgkmcnt0();
        store_staged_fused<OUT_BF16, DEBUG>(stf, OPF, SH, WTN, m0 + wm * WTM + 16 * i, n0 + wn * WTN,
                                            lane, 64, eo);
        wait_lgkmcnt0();
      }
    }
    wait_lgkmcnt0();
    block_barrier();
  }
}

}  // namespace tg
