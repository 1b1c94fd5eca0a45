// mx_kernel.hpp -- microscaled FP8 / FP4 (MXFP8, MXFP4) tile kernel for gfx950.
//
// The low-precision GEMMs the TorchInductor page measures beside bf16
// ("TorchInductor ganha suporte a GEMMs de alta performance com CuteDSL", its
// MXFP8 benchmark paragraph), read as the OCP MX format: E4M3 elements, one
// E8M0 scale per 32 consecutive elements along K. A is M x K (row-major,
// bytes), B is given as its N x K transpose (K-contiguous), scales are
// row-major [rows][ls] bytes with ls >= K / 32 a multiple of 4.
//
// Partition and ownership are the tile kernel's: every BM x BN output tile is
// owned by one workgroup (a persistent grid walks tiles wg, wg + grid, ...),
// which reads A and B as shared immutable views and writes its tile once.
// A slab is 64 K values = 64 bytes per row, the same LDS row as the bf16
// kernel's 32-element slab, so staging (direct buffer -> LDS loads through
// range-checked resources), the swizzled layout and the operand reads are
// those of the tile kernel. Each 64-K slab is one v_mfma_scale_f32_32x32x64
// per 32 x 32 block: lane l holds row (l % 32), bytes 0-15 from the slab's
// first 32-element block and bytes 16-31 from its second (LDS chunks l / 32
// and 2 + l / 32), and the scale of block b of row r sits in lane r + 32 b
// (measured on the device with a one-wave probe). Each lane therefore needs
// the scale of its row for block 2 s + l / 32: one dword of the scale row
// covers two slabs; it is shifted by 8 (l / 32) bits per lane and the
// instruction's byte select picks byte 0 or 2 by slab parity. Scales travel
// like the operands: 16 bytes of every row of the tile (the scales of 8
// slabs) are loaded straight into a ring of LDS windows together with the
// first slab they cover, so their loads are ordered with the slabs' and need
// no wait of their own. Row r of a window starts g = (r / 8) % 4 dwords
// later in its scale row (window w holds its dwords 4 w + g .. 4 w + g + 3,
// and a window -1 the first g), so one 4-byte read of dword d of 32 rows, 16
// bytes apart, takes it from position (d - g) % 4 of window w or w - 1: rows
// that share a bank group (r, r + 8, r + 16, r + 24) read four different
// positions, and the 32 reads fall in 32 banks instead of 8 banks four times.
//
// MXFP4 (E2M1, two elements per byte, the lower K index in the low nibble)
// uses the same 64-byte rows, now 128 K values per slab: each 16-byte LDS
// chunk is one 32-element block and one instruction operand, so a slab is two
// instructions per 32 x 32 block (chunks l / 32, then 2 + l / 32), and a scale
// dword covers one slab (byte 2 m + l / 32 for its instruction m).
//
// K advances in ascending order (fp32 accumulation, no split-K), so results
// are bit-identical run to run.
#pragma once

#include "tile_kernel.hpp"

namespace tg {

struct MxArgs {
  const uint8_t* A;   // M x K E4M3, lda bytes between rows
  const uint8_t* B;   // N x K E4M3 (B transposed), ldb bytes between rows
  const uint8_t* sA;  // M x ls E8M0
  const uint8_t* sB;  // N x ls E8M0
  void* C;
  int32_t M, N, K;
  int64_t lda, ldb, ldc;
  int32_t ls;  // scale row stride in bytes (multiple of 4)
  TileMap map;
  uint32_t* counts;  // debug instrumentation only
  int32_t flags;
  const float* bias;
  int32_t act;
};

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// Element formats of the MX kernel (the C ABI's tile_gemm_mx_format_t).
constexpr int kMxE4M3 = 0, kMxE2M1 = 1;

// One 32 x 32 x 64 scaled step of a C block held transposed (as mma()): the B
// fragment is the instruction's first operand. OPSEL picks the scale byte;
// HW is the instruction's element-format code (0 E4M3, 4 E2M1).
template <int OPSEL, int HW>
__device__ __forceinline__ floatx16 mma_mx(const i32x8& a_frag, const i32x8& b_frag, int a_scale,
                                           int b_scale, const floatx16& acc) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b_frag, a_frag, acc, HW, HW, OPSEL,
                                                         b_scale, OPSEL, a_scale);
}

// The 16 bytes of half H (0: LDS chunk l / 32, 1: chunk 2 + l / 32) of a
// staged fragment as an E2M1 operand: 32 four-bit elements, one MX block.
template <int H>
__device__ __forceinline__ i32x8 fp4_half(const i32x8& f) {
  if constexpr (H == 0) return i32x8{f[0], f[1], f[2], f[3], 0, 0, 0, 0};
  else return i32x8{f[4], f[5], f[6], f[7], 0, 0, 0, 0};
}

template <int BM, int BN, int WM, int WN, int NST, int FMT, bool OUT_BF16, bool DEBUG>
__global__ __launch_bounds__(WM * WN * 64, 1) void mx_gemm_kernel(MxArgs p) {
  static_assert(NST >= 4 && NST <= 12, "ring depth");
  static_assert(FMT == 0 || FMT == 1, "E4M3 or E2M1 elements");
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  constexpr bool FP4 = FMT == kMxE2M1;
  constexpr int HW = FP4 ? 4 : 0;         // the instruction's format code
  constexpr int BKB = 64;                 // bytes per row and slab
  constexpr int KPS = FP4 ? 128 : 64;     // K elements per slab
  constexpr int SPW = FP4 ? 4 : 8;        // slabs per scale window (16 scale bytes per row)
  constexpr int A_BYTES = BM * BKB;
  constexpr int B_BYTES = BN * BKB;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_DMA = A_BYTES / 1024, B_DMA = B_BYTES / 1024;
  static_assert(A_DMA % NW == 0 && B_DMA % NW == 0, "slabs split evenly over the waves");
  constexpr int A_PER = A_DMA / NW, B_PER = B_DMA / NW;
  constexpr int NDMA = A_PER + B_PER;     // DMA instructions per wave and slab
  constexpr int RING = NST * STAGE;
  constexpr int SWIN = (BM + BN) * 16;    // one scale window: 16 bytes per row
  // Window w lives in buffer (w + 1) % NWB (window -1 in buffer 0). Window w
  // + NWB - 1 reuses window w - 1's buffer. It goes out with slab SPW (w + NWB
  // - 1), at step SPW (w + NWB - 1) - NST at the earliest, after that step's
  // barrier; the last read of window w - 1's buffer is the take of window w's
  // third dword (rows with g = 3), at the start of step SPW w + T1.
  constexpr int T1 = FP4 ? 2 : 4;
  constexpr int NWB = 1 + (NST + T1 + SPW - 1) / SPW;
  static_assert(SPW * (NWB - 1) - NST >= T1, "a scale window is reloaded only after its last use");
  static_assert(BM % 64 == 0 && BN % 64 == 0, "scale windows are whole KiB per wave instruction");
  constexpr int SA_DMA = BM / 64, SB_DMA = BN / 64;   // window loads (1 KiB each)

  __shared__ __attribute__((aligned(1024))) uint4 smem[(RING + NWB * SWIN) / 16];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave - (wave / WN) * WN;
  const int lrow = lane & 31, lgrp = lane >> 5;
  const int M = p.M, N = p.N, K = p.K;
  const int64_t lda = p.lda, ldb = p.ldb;
  const int nk = K / KPS;                 // K is a multiple of KPS
  const int kbytes = FP4 ? K / 2 : K;     // bytes of K in a row

  // per-lane DMA source offsets within a slab (bytes), fixed for the kernel
  uint32_t voA[A_PER], voB[B_PER];
#pragma unroll
  for (int t = 0; t < A_PER; ++t) {
    const int r = 16 * (wave + NW * t) + (lane >> 2);
    voA[t] = (uint32_t)(r * lda) + (((lane & 3) ^ swzA(r)) << 4);
  }
#pragma unroll
  for (int t = 0; t < B_PER; ++t) {
    const int r = 16 * (wave + NW * t) + (lane >> 2);
    voB[t] = (uint32_t)(r * ldb) + (((lane & 3) ^ swzA(r)) << 4);
  }
  const uint32_t ldsw = __builtin_amdgcn_readfirstlane(lds0 + 1024 * wave);
  // this lane's LDS read addresses of stage 0 (chunk lgrp and 2 + lgrp)
  const int swl = (lrow >> 2) & 3;
  const uint32_t rA0 = lds0 + (wm * WTM + lrow) * 64 + (((lgrp ^ swl)) << 4);
  const uint32_t rA1 = lds0 + (wm * WTM + lrow) * 64 + (((lgrp ^ swl) ^ 2) << 4);
  const uint32_t rB0 = lds0 + A_BYTES + (wn * WTN + lrow) * 64 + (((lgrp ^ swl)) << 4);
  const uint32_t rB1 = lds0 + A_BYTES + (wn * WTN + lrow) * 64 + (((lgrp ^ swl) ^ 2) << 4);

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

    const int sh = 8 * lgrp;
    // scale windows: rows of both scale arrays with exact extents (rows past
    // the edge read as zero and are never used)
    const i32x4 rsSA = make_rsrc(p.sA, (int64_t)M * p.ls);
    const i32x4 rsSB = make_rsrc(p.sB, (int64_t)N * p.ls);
    const uint32_t swin0 = lds0 + RING;
    // Load window w (16 bytes of each of the tile's rows: the scales of slabs
    // SPW w .. SPW w + SPW - 1, from 4 g bytes later for row r, g = (r / 8) %
    // 4) into buffer (w + 1) % NWB: instruction q covers rows 64 q ..; of
    // window -1 only the first g dwords of each row are ever read (rows with
    // g = 0 load their row's first bytes instead of reaching before it).
    auto issue_window = [&](int w) {
      const uint32_t dst = swin0 + (uint32_t)(((w + 1) % NWB) * SWIN);
      // the byte of its scale row this lane starts at (window -1, g > 0:
      // 4 g - 16, inside the row before, as such a row is never the first)
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

    // The window of slabs SPW w .. goes out just before slab SPW w's own loads,
    // so any wait that covers slab SPW w covers it too.
    auto issue_slab = [&](int s) {
      if (s % SPW == 0) issue_window(s / SPW);
      const uint32_t st = (uint32_t)(s % NST) * STAGE;
      const i32x4 rsA = make_rsrc(a_panel + (int64_t)s * BKB, a_bytes - (int64_t)s * BKB);
      const i32x4 rsB = make_rsrc(b_panel + (int64_t)s * BKB, b_bytes - (int64_t)s * BKB);
#pragma unroll
      for (int t = 0; t < A_PER; ++t) dma16(ldsw + st + 1024 * NW * t, rsA, voA[t], 0u);
#pragma unroll
      for (int t = 0; t < B_PER; ++t) dma16(ldsw + st + A_BYTES + 1024 * NW * t, rsB, voB[t], 0u);
    };
    // wait until this wave's loads of slab s have landed, given the slabs
    // issued after it (0 .. NST - 1 of them; whole slabs only: scale loads
    // make the real count larger, so this waits at least as long as needed)
    auto wait_after = [&](int after) {
      static_for<0, NST>([&](auto a_c) {
        constexpr int a = decltype(a_c)::value;
        if (after == a) wait_vmcnt<a * NDMA>();
      });
    };

    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = floatx16{};

    i32x8 af[2][FM], bfr[2][FN];
    // scales of slab s in set s % 2, shifted per lane: the set a take writes
    // is never the one the MFMAs still in flight read
    int sca[2][FM], scb[2][FN];
    uint32_t rsa[FM], rsb[FN];  // their scale dwords, read a step ahead
    // this lane's first A and B rows in a scale window (bytes)
    const uint32_t sra = (uint32_t)((wm * WTM + lrow) * 16);
    const uint32_t srb = (uint32_t)(BM * 16 + (wn * WTN + lrow) * 16);
    auto read_frags = [&](int s, int slot) {
      const uint32_t so = (uint32_t)(s % NST) * STAGE;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint4 x = __builtin_bit_cast(uint4, lds_read16(rA0 + so + i * 2048));
        const uint4 y = __builtin_bit_cast(uint4, lds_read16(rA1 + so + i * 2048));
        af[slot][i] = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint4 x = __builtin_bit_cast(uint4, lds_read16(rB0 + so + j * 2048));
        const uint4 y = __builtin_bit_cast(uint4, lds_read16(rB1 + so + j * 2048));
        bfr[slot][j] = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
      }
    };
    // Scales from window s / SPW, landed with its first slab before the
    // barrier that made that slab readable. A scale dword is read one step
    // before the first step that takes it (after that step's barrier), so the
    // read latency never stands before an MFMA; every step takes (shifts) its
    // slab's scales into the register set of its parity. E4M3: the dword of
    // slabs s, s + 1 (s even), read once for both, byte 2 (s % 2) + l / 32
    // after the shift; E2M1: the dword of slab s (its four blocks), byte
    // 2 m + l / 32 for the slab's MFMA m.
    auto fetch_scales = [&](int s) {
      const int w = s / SPW;
      const int dw = FP4 ? (s % SPW) : ((s % SPW) >> 1);
      // dword dw of a row with g = (row / 8) % 4 (row = 32 k + lrow): position
      // (dw - g) % 4 of window w, or of window w - 1 when dw < g
      const int g = (lrow >> 3) & 3;
      const int buf = dw < g ? w : w + 1;
      const uint32_t wb = swin0 + (uint32_t)((buf % NWB) * SWIN) + (uint32_t)(4 * ((dw - g) & 3));
      // one address per operand; the fragments' rows are constant offsets
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
    // MFMA k of a slab (k < NMFMA): block (i, j) and, for E2M1, half m
    constexpr int NBLK = FM * FN;
    constexpr int NMFMA = FP4 ? 2 * NBLK : NBLK;
    auto mfma_k = [&](auto k_c, auto par_c, int slot) {
      constexpr int k = decltype(k_c)::value, PAR = decltype(par_c)::value;
      constexpr int b = k % NBLK, i = b / FN, j = b % FN;
      if constexpr (FP4) {
        constexpr int m = k / NBLK;
        acc[i][j] = mma_mx<2 * m, HW>(fp4_half<m>(af[slot][i]), fp4_half<m>(bfr[slot][j]), sca[PAR][i],
                                      scb[PAR][j], acc[i][j]);
      } else {
        acc[i][j] = mma_mx<2 * PAR, HW>(af[slot][i], bfr[slot][j], sca[PAR][i], scb[PAR][j], acc[i][j]);
      }
    };
    // Step s: slab s's operands are in registers (slot s % 2). At its start
    // the wave waits for slab s + 1's loads and for its own reads of slab s
    // (issued last step), then one barrier: every wave has slab s in
    // registers, so slab s's stage takes slab s + NST, and slab s + 1 may be
    // read. Slab s's MFMAs then run with slab s + 1's operand reads and slab
    // s + NST's loads spread evenly among them, so neither the LDS nor the
    // texture unit sees a burst.
    constexpr int NUNIT = FM + FN;  // operand units: A fragment u < FM, else B fragment u - FM
    auto read_unit = [&](uint32_t so, int slot, auto idx_c) {
      constexpr int IDX = decltype(idx_c)::value;
      if constexpr (IDX < FM) {
        const uint4 x = __builtin_bit_cast(uint4, lds_read16(rA0 + so + IDX * 2048));
        const uint4 y = __builtin_bit_cast(uint4, lds_read16(rA1 + so + IDX * 2048));
        af[slot][IDX] = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
      } else {
        const uint4 x = __builtin_bit_cast(uint4, lds_read16(rB0 + so + (IDX - FM) * 2048));
        const uint4 y = __builtin_bit_cast(uint4, lds_read16(rB1 + so + (IDX - FM) * 2048));
        bfr[slot][IDX - FM] =
            i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
      }
    };
    // DMA unit t of a slab (t < A_PER: this wave's A load t, else its B load
    // t - A_PER) into the stage at byte offset st.
    auto dma_unit = [&](uint32_t st, const i32x4& rsA, const i32x4& rsB, auto t_c) {
      constexpr int t = decltype(t_c)::value;
      if constexpr (t < A_PER)
        dma16(ldsw + st + 1024 * NW * t, rsA, voA[t], 0u);
      else
        dma16(ldsw + st + A_BYTES + 1024 * NW * (t - A_PER), rsB, voB[t - A_PER], 0u);
    };
    // the MFMA after which operand unit u, and DMA unit t, are issued
    auto read_slot = [](int u) constexpr { return ((2 * u + 1) * NMFMA) / (2 * NUNIT); };
    auto dma_slot = [](int t) constexpr { return ((2 * t + 1) * NMFMA) / (2 * NDMA); };
    static_assert(NST >= 2 && (NST - 1) * NDMA <= 63, "loads in flight fit the counter");
    // Steady step (slab s + NST exists, so NST - 2 whole slabs follow s + 1)
    auto step_full = [&](int s, auto par_c) {
      constexpr int PAR = decltype(par_c)::value;  // s % 2
      take_scales(PAR);
      wait_vmcnt<(NST - 2) * NDMA>();
      wait_lgkmcnt0();
      block_barrier();
      if (FP4 || PAR == 1) fetch_scales(s + 1);
      const int sn = s + NST;
      if (sn % SPW == 0) issue_window(sn / SPW);
      const uint32_t stn = (uint32_t)(sn % NST) * STAGE;
      const i32x4 rsA = make_rsrc(a_panel + (int64_t)sn * BKB, a_bytes - (int64_t)sn * BKB);
      const i32x4 rsB = make_rsrc(b_panel + (int64_t)sn * BKB, b_bytes - (int64_t)sn * BKB);
      const uint32_t so = (uint32_t)((s + 1) % NST) * STAGE;
      __builtin_amdgcn_sched_barrier(0);
      // (a fence after each MFMA and what goes with it: the loads are inline
      // assembly, which the scheduler would otherwise gather into one burst)
      static_for<0, NMFMA>([&](auto k_c) {
        constexpr int k = decltype(k_c)::value;
        mfma_k(k_c, par_c, PAR);
        static_for<0, NUNIT>([&](auto u_c) {
          if constexpr (read_slot(decltype(u_c)::value) == k) read_unit(so, PAR ^ 1, u_c);
        });
        static_for<0, NDMA>([&](auto t_c) {
          if constexpr (dma_slot(decltype(t_c)::value) == k) dma_unit(stn, rsA, rsB, t_c);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    // Any step, near the end of K: the same order, with the waits counted
    // from the slabs that exist and slab s + NST's loads (if it exists) in
    // one burst after the barrier.
    auto step = [&](int s, auto par_c) {
      constexpr int PAR = decltype(par_c)::value;
      take_scales(PAR);
      if (s + 1 < nk) wait_after((nk - 1 < s + NST - 1 ? nk - 1 : s + NST - 1) - (s + 1));
      wait_lgkmcnt0();
      block_barrier();
      // (after the last slab: dwords of a buffer in bounds, never used)
      if (FP4 || PAR == 1) fetch_scales(s + 1);
      if (s + NST < nk) issue_slab(s + NST);
      const uint32_t so = (uint32_t)((s + 1) % NST) * STAGE;
      __builtin_amdgcn_sched_barrier(0);
      // unconditional, after the last slab too: it then reads a stale stage
      // (in bounds) whose values are never used
      static_for<0, NMFMA>([&](auto k_c) {
        constexpr int k = decltype(k_c)::value;
        mfma_k(k_c, par_c, PAR);
        static_for<0, NUNIT>([&](auto u_c) {
          if constexpr (read_slot(decltype(u_c)::value) == k) read_unit(so, PAR ^ 1, u_c);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    // prologue: slabs 0 .. NST - 1 in flight, slab 0 landed and read
    const int n_full = nk - NST;  // steady steps: slab s + NST exists
    if (nk > 0) {
      issue_window(-1);
      for (int sl = 0; sl < NST && sl < nk; ++sl) issue_slab(sl);
      wait_after((nk - 1 < NST - 1 ? nk - 1 : NST - 1));
      block_barrier();
      read_frags(0, 0);
      fetch_scales(0);
    }
    // Steps run in pairs (the register slot of slab s is s % 2).
    int s = 0;
    const std::integral_constant<int, 0> p0{};
    const std::integral_constant<int, 1> p1{};
    for (; s + 2 <= n_full; s += 2) {
      step_full(s, p0);
      step_full(s + 1, p1);
    }
    if (s < n_full) {  // an odd number of steady steps: the last one, then realign
      step_full(s, p0);
      ++s;
      if (s < nk) step(s++, p1);
    }
    for (; s + 2 <= nk; s += 2) {
      step(s, p0);
      step(s + 1, p1);
    }
    if (s < nk) step(s, p0);

    // Store: the summed tile is staged in the free ring as fp32 strips and
    // written once per element (with the fused epilogue when asked).
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
