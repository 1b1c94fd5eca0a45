// tile16_kernel.hpp -- the LDS-staged tile kernel on 16x16x32 bf16 MFMA blocks.
//
// Ownership, staging and the LDS layouts are those of tile_kernel.hpp (every
// BM x BN tile has one owning workgroup, its only writer; 32-wide K slabs
// reach LDS by direct buffer-to-LDS loads through a ring of NST stages; A and
// a column-major B are stored K-contiguous in 64-byte rows with chunk
// swizzling -- by other row bits, see swz16 -- a row-major B N-contiguous and
// read transposed). What differs is
// the matrix instruction: v_mfma_f32_16x16x32_bf16 instead of the 32x32x16
// form. Measured on gfx950 with random operands, two waves per SIMD issue the
// 32x32x16 instruction at about 61% of the MFMA pipe's rate while the
// 16x16x32 one keeps it about 95% busy (at a higher sustained clock), so the
// eight-wave tiles run on 16x16 blocks.
//
// One 16x16x32 MFMA consumes a whole 32-wide slab for a 16 x 16 block: lane l
// supplies row (l % 16) of the A block and column (l % 16) of the B block,
// each as the 8 values of k chunk (l / 16), i.e. one 16-byte LDS read per
// lane per block. The B fragment goes in as the instruction's row operand and
// the A fragment as its column operand, so the block of C comes out
// transposed: lane l holds C row (l % 16), columns 4 (l / 16) .. + 3 -- four
// consecutive columns of one row, which the epilogue stages and stores as
// row chunks. Each output element is the fp32 sum of its K products taken
// slab by slab in ascending K, one instruction per slab.
//
// Per wave and slab s the FM x FN blocks of its WTM x WTN sub-tile are taken
// in NSTEP = FM / 2 steps of two A block rows each:
//   steps 0 .. NSTEP-2: their blocks, while reading the next step's two A
//           fragments and issuing the second half of this wave's loads of
//           slab s + NST - 2 (into the stage the previous barrier freed);
//   wait for this wave's loads of slab s + 1, barrier (every wave's loads of
//   s + 1 have landed and every wave is done reading s - 1);
//   step NSTEP-1: its blocks column by column, while reading the next slab's
//           first two A fragments, and each B fragment of the next slab right
//           after the last MFMA that uses this slab's one, and issuing the
//           first half of the loads of slab s + NST - 1 into the stage s - 1
//           just freed.
// The A fragments alternate between two small register sets; the B fragments
// are held once. With 128 x 64 wave tiles that keeps the eight-wave kernel
// within the 256 registers a wave has at two waves per SIMD.
#pragma once

#include "tile_kernel.hpp"

namespace tg {

// Chunk swizzle of the K-contiguous layout (A, column-major B): 16-byte
// chunk c of slab row r sits at position c ^ swz16(r) of its 64-byte row.
// A fragment read covers 16 consecutive rows and all four chunks; measured
// with the kernel's own read sequences on gfx950 (bank-conflict and LDS-busy
// counters), XOR with bits 1-2 of the row makes those reads conflict-free,
// while bits 2-3 (the 32x32x16 kernel's choice, whose reads cover 32 rows of
// one chunk) or bits 0-1 double the LDS cycles per read.
__device__ __forceinline__ int swz16(int r) { return (r >> 1) & 3; }

// Chunk placement of a row-major B slab (k rows of CPR 16-byte chunks):
// chunk c of k row r sits at position swzB<CPR>(c, r) of its row. A B
// fragment is two transposing 8-byte reads; each 16 lanes of one read take
// 32 bytes (two chunks) from each of four consecutive k rows, which must land
// in four different 32-byte bank groups. The rows' chunks are XORed in
// aligned groups (so each group stays in place and the map is its own
// inverse): the first CPR & ~15 chunks with (r % 4) in bits 1-2 and bit 3 of
// r in bit 3, the next aligned 8 with (r % 4) in bits 1-2, and an aligned 4
// that follows (rows then start 64 bytes apart mod 128) with bit 1 of r in
// bit 1. Any chunks after those stay in place.
template <int CPR>
__device__ __forceinline__ int swzB(int c, int r) {
  constexpr int GA = CPR >= 16 ? (CPR & ~15) : 0, GB = CPR & ~7, GC = CPR & ~3;
  if (c < GA) return c ^ (((r & 3) << 1) | (((r >> 3) & 1) << 3));
  if (c < GB) return c ^ ((r & 3) << 1);
  if (c < GC) return c ^ (((r >> 1) & 1) << 1);
  return c;
}

// 16 x 16 x 32 step of a C block held transposed (see above), accumulated in
// place. With one wave per SIMD the 128 x 128 wave tiles hold 256
// accumulator values, the whole accumulation-register file: there the
// compiler's own form of the instruction (destination distinct from the
// accumulator input) makes it move every accumulator every few MFMAs, so the
// instruction is written out with its accumulator tied in place. The compiler
// does not see an MFMA in it, so the kernel keeps the instruction's hazards
// itself: a vector ALU write of an operand (the accumulators' zeroing, a
// register copy) needs two wait states before the MFMA reads it, issued by
// tied_entry() at the head of every K loop iteration (the fragments inside an
// iteration come straight from LDS reads; a check of the built code's MFMAs
// against the vector ALU writes before them guards this), and settle_tied()
// waits out the result latency before the accumulators are read.
template <bool TIED>
__device__ __forceinline__ void mma16(floatx4& acc, const bf16x8& a_frag, const bf16x8& b_frag) {
  if constexpr (TIED)
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(b_frag), "v"(a_frag));
  else
    acc = mfma16(b_frag, a_frag, acc);
}
__device__ __forceinline__ void tied_entry() { asm volatile("s_nop 1"); }

// Before the accumulators of written-out MFMAs (mma16<true>) are read: wait
// out the last MFMA's result latency (32 wait states, more than any MFMA form
// needs before another instruction reads its result), then tie accumulators
// to a point after the wait so that no read moves above it: all of them at
// once (settle_tied(acc)), or a block row right before the epilogue takes it
// (pin_row), which also keeps the reads of later rows from moving ahead --
// reading all 256 values at once needs more registers than a wave has, and
// the compiler then spills. Which of the two a kernel uses is fixed by what
// its build passes in the hazard check: given the freedom of row pins, the
// 32-deep 256 x 256 kernel's allocator moved accumulators through vector
// registers inside its K loop.
__device__ __forceinline__ void settle_tied() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"); }
template <int FM, int FN>
__device__ __forceinline__ void settle_tied(floatx4 (&acc)[FM][FN]) {
  settle_tied();
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) asm volatile("" : "+a"(acc[i][j]));
}
template <int FN>
__device__ __forceinline__ void pin_row(floatx4 (&row)[FN]) {
#pragma unroll
  for (int j = 0; j < FN; ++j) asm volatile("" : "+a"(row[j]));
}

template <int BM, int BN, int WM, int WN, int NST, bool BCOL, bool OUT_BF16, bool DEBUG>
__global__ __launch_bounds__(WM * WN * 64, 1) void tile16_gemm_kernel(TileArgs p) {
  constexpr int kStages = NST;
  static_assert(NST >= 3 && NST <= 6, "ring depth");
  constexpr int NW = WM * WN;
  constexpr int NT = NW * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int FQ = 2;             // A blocks (16-row) per step
  constexpr int NSTEP = FM / FQ;    // steps per slab
  constexpr int NM = FQ * FN;       // MFMAs per step
  constexpr int RB = BCOL ? 1 : 2;  // LDS instructions per B fragment
  static_assert(WTM % (32 * FQ) == 0 && WTN % 16 == 0,
                "wave tile: an even number of steps of FQ 16-row blocks, whole 16-column blocks");
  static_assert(NW == 4 || NW == 8, "one or two waves per SIMD");
  constexpr bool TIED = NW == 4;  // accumulators tied in place (see mma16)
  constexpr int BK = kTileBK;
  constexpr int A_BYTES = BM * BK * 2;  // per stage
  constexpr int B_BYTES = BN * BK * 2;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_DMA = A_BYTES / 1024;  // one KiB per wave instruction
  constexpr int B_DMA = B_BYTES / 1024;
  static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "slabs are whole KiB");
  static_assert(A_DMA % NW == 0, "A slab splits evenly over the waves");
  static_assert(STAGE + 16 * 1024 <= 65536, "ds_read immediate offsets within a stage pair");
  constexpr int A_PER = A_DMA / NW;
  constexpr int B_MAX = (B_DMA + NW - 1) / NW;
  constexpr int B_MIN = B_DMA / NW;
  constexpr int PITCH = BN * 2;  // row-major B: bytes per k row
  constexpr int CPR = BN / 8;  // row-major B: 16-byte chunks per k row

  __shared__ __attribute__((aligned(1024))) uint4 smem[kStages * STAGE / 16];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave - (wave / WN) * WN;
  const int l16 = lane & 15, lg = lane >> 4;  // block row / column, k chunk
  // row-major B transposed reads: lane = 16 G + 4 j + q
  const int tG = lane >> 4, tj = (lane >> 2) & 3, tq = lane & 3;

  const int n_tiles = p.map.tiles_m * p.map.tiles_n;
  for (int wg_it = blockIdx.x; wg_it < n_tiles; wg_it += gridDim.x) {
    int wg = wg_it;
    if constexpr (DEBUG) {
      if ((p.flags & kDbgCollide) && wg == 1) wg = 0;  // negative control only
    }
    int32_t tm, tn;
    tile_of(p.map, wg, tm, tn);
    // With the accumulators tied, the compiler's count of outstanding vector
    // memory operations carries the last tile's epilogue into the K loop and
    // it drains every load at the loop's head; settled here, once per tile,
    // the loop keeps only its own waits.
    if constexpr (TIED) wait_vmcnt<0>();
    const int M = p.M, N = p.N, K = p.K;
    const int64_t lda = p.lda, ldb = p.ldb;
    const int glu = p.glu_half;
    const int gshift = glu ? glu - BN / 2 : 0;
    const int m0 = tm * BM, n0 = tn * (glu ? BN / 2 : BN);

    // ---- panels, their valid extents (to the operand's last element), steps
    const char* a_panel = reinterpret_cast<const char*>(p.A + (int64_t)m0 * lda);
    const int64_t a_bytes = K > 0 ? (((int64_t)(M - 1) * lda + K) - (int64_t)m0 * lda) * 2 : 0;
    const char* b_panel = reinterpret_cast<const char*>(BCOL ? p.B + (int64_t)n0 * ldb : p.B + n0);
    const int64_t b_bytes = K <= 0 ? 0
                            : BCOL ? (((int64_t)(N - 1) * ldb + K) - (int64_t)n0 * ldb) * 2
                                   : (((int64_t)(K - 1) * ldb + N) - n0) * 2;
    const int64_t a_step = BK * 2;
    const int64_t b_step = BCOL ? BK * 2 : BK * ldb * 2;

    // ---- per-lane DMA source offsets (bytes), fixed for the whole K loop
    uint32_t voA[A_PER];
#pragma unroll
    for (int t = 0; t < A_PER; ++t) {
      const int ins = wave + NW * t;
      const int r = 16 * ins + (lane >> 2);
      const int c = (lane & 3) ^ swz16(r);
      voA[t] = (uint32_t)(r * lda * 2) + c * 16;
    }
    const int b_cnt = (wave < B_DMA % NW) ? B_MAX : B_MIN;
    uint32_t voB[B_MAX];
#pragma unroll
    for (int t = 0; t < B_MAX; ++t) {
      const int ins = wave + NW * t;
      if constexpr (BCOL) {
        const int r = 16 * ins + (lane >> 2);
        const int c = (lane & 3) ^ swz16(r);
        voB[t] = (uint32_t)((r + (r >= BN / 2 ? gshift : 0)) * ldb * 2) + c * 16;
      } else {
        const int q = 64 * ins + lane;
        const int row = q / CPR, pc = q - (q / CPR) * CPR;
        const int lc = swzB<CPR>(pc, row);  // the chunk that belongs at position pc
        voB[t] = (uint32_t)(row * ldb * 2) + lc * 16 + (lc >= CPR / 2 ? 2 * gshift : 0);
      }
    }

    const int nk = (K + BK - 1) / BK;
    // Slabs loaded by DMA; the rest (a K tail, and with a row-major B and an
    // odd N the slab holding B's last value, whose dword straddles the end of
    // the resource and would read as zero) go through registers.
    const int nk_full = (!BCOL && (N & 1)) ? (K - 1) / BK : K / BK;

    auto issue_slab = [&](int s) {
      const int st = s % kStages;
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
        // exact zeros past K (and past M, N) in both operands, through registers
        const int k0 = s * BK;
        uint4* dA = reinterpret_cast<uint4*>(reinterpret_cast<char*>(smem) + st * STAGE);
        uint4* dB = reinterpret_cast<uint4*>(reinterpret_cast<char*>(smem) + st * STAGE + A_BYTES);
        for (int q = tid; q < BM * 4; q += NT) {
          const int r = q >> 2, c = q & 3;
          const uint4 v = (m0 + r < M) ? load8_masked(p.A + (int64_t)(m0 + r) * lda, k0 + 8 * c, K)
                                       : make_uint4(0, 0, 0, 0);
          dA[r * 4 + (c ^ swz16(r))] = v;
        }
        if constexpr (BCOL) {
          for (int q = tid; q < BN * 4; q += NT) {
            const int r = q >> 2, c = q & 3;
            const int col = n0 + r + (r >= BN / 2 ? gshift : 0);
            const uint4 v = (col < N) ? load8_masked(p.B + (int64_t)col * ldb, k0 + 8 * c, K)
                                      : make_uint4(0, 0, 0, 0);
            dB[r * 4 + (c ^ swz16(r))] = v;
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

    // DMA units [lo, hi) of full slab s: units 0 .. A_PER-1 are this wave's A
    // loads, then its b_cnt B loads.
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
        if (t < b_cnt && A_PER + t >= lo && A_PER + t < hi)
          dma16(lb + 1024 * (wave + NW * t), rsB, voB[t], 0u);
    };

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

    floatx4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{};

    // ---- LDS read addresses. Lane bases per stage pair (a ds_read immediate
    // reaches 64 KiB, two stages plus the block offsets); swz16 of a block row
    // depends only on the row within its 16-row block.
    constexpr int NPAIR = (kStages + 1) / 2;
    const uint32_t chunk = (uint32_t)((lg ^ swz16(l16)) << 4);
    uint32_t rA[NPAIR], rB[NPAIR];
#pragma unroll
    for (int h = 0; h < NPAIR; ++h) {
      rA[h] = lds0 + 2 * h * STAGE + (uint32_t)((wm * WTM + l16) * 64) + chunk;
      rB[h] = lds0 + 2 * h * STAGE + A_BYTES + (uint32_t)((wn * WTN + l16) * 64) + chunk;
    }
    uint32_t rT[BCOL ? 1 : FN][NPAIR];  // row-major B: per block and stage pair
#pragma unroll
    for (int j = 0; j < (BCOL ? 1 : FN); ++j) {
      // rows 8 G + j and 8 G + 4 + j share their chunk placement
      const int n = wn * WTN + 16 * j + 4 * tq;
      const int col = (swzB<CPR>(n >> 3, 8 * tG + tj) << 3) | (n & 7);
      const uint32_t b = lds0 + A_BYTES + (uint32_t)((8 * tG + tj) * PITCH + col * 2);
#pragma unroll
      for (int h = 0; h < NPAIR; ++h) rT[j][h] = b + 2 * h * STAGE;
    }

    bf16x8 aS[2][FQ];  // A fragments: step q uses set q & 1 while set (q + 1) & 1 is read
    bf16x8 bq[FN];     // B fragments of the current slab

    // A block I of the slab in stage ST
    auto readA = [&](auto st_c, auto i_c) -> bf16x8 {
      constexpr int ST = decltype(st_c)::value, I = decltype(i_c)::value;
      return lds_read16(rA[ST >> 1] + (uint32_t)((ST & 1) * STAGE + I * 1024));
    };
    // B block J of the slab in stage ST
    auto readB = [&](auto st_c, auto j_c) -> bf16x8 {
      constexpr int ST = decltype(st_c)::value, J = decltype(j_c)::value;
      if constexpr (BCOL) {
        return lds_read16(rB[ST >> 1] + (uint32_t)((ST & 1) * STAGE + J * 1024));
      } else {
        const uint32_t b = rT[J][ST >> 1] + (uint32_t)((ST & 1) * STAGE);
        const i16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(uintptr_t)(b));
        const i16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(uintptr_t)(b + 4 * PITCH));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    // The same reads with a run-time stage (general loop and prologue).
    auto readA_rt = [&](int st, int i) -> bf16x8 {
      return lds_read16(lds0 + st * STAGE + (uint32_t)((wm * WTM + l16) * 64) + chunk + i * 1024);
    };
    auto readB_rt = [&](int st, int j) -> bf16x8 {
      if constexpr (BCOL) {
        return lds_read16(lds0 + st * STAGE + A_BYTES + (uint32_t)((wn * WTN + l16) * 64) + chunk +
                          j * 1024);
      } else {
        const uint32_t b = rT[j][0] + (uint32_t)(st * STAGE);
        const i16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(uintptr_t)(b));
        const i16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(uintptr_t)(b + 4 * PITCH));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };

    const int n_steady = nk_full - (kStages - 1);
    const bool split = n_steady >= kStages;
    const int ndma = A_PER + b_cnt;
    const int nh1 = (ndma + 1) / 2;

    // ---- prologue: slabs 0..kStages-2 in flight (the last one only its first
    // half when the steady loop runs), slab 0 ready, its step-0 operands read
    if (nk > 0) {
#pragma unroll
      for (int s = 0; s < kStages - 1; ++s) {
        if (s < nk) {
          if (split && s == kStages - 2) issue_units(s, 0, nh1);
          else issue_slab(s);
        }
      }
      if (split) {
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
#pragma unroll
      for (int f = 0; f < FQ; ++f) aS[0][f] = readA_rt(0, f);
#pragma unroll
      for (int j = 0; j < FN; ++j) bq[j] = readB_rt(0, j);
    }

    // Order of a step's MFMAs: the last step of a slab goes column by column,
    // so B fragment j of the next slab can be read right after the last MFMA
    // that uses this slab's fragment j; the other steps row by row.
    auto blk = [](int q, int k) constexpr {
      return q == NSTEP - 1 ? (k % FQ) * FN + (k / FQ) : k;   // i * FN + j within the step
    };
    // LDS read instructions issued right after MFMA k of step q (the pattern
    // the scheduler is held to): in steps before the last, A fragment f of the
    // next step after MFMA f * NM / FQ; in the last step, the next slab's A
    // fragments after MFMAs 0 .. FQ - 1 and B fragment j after the last MFMA
    // of column j.
    auto nreads = [](int q, int k) constexpr {
      if (q != NSTEP - 1) return (k * FQ) % NM == 0 ? 1 : 0;
      return (k < FQ ? 1 : 0) + (k % FQ == FQ - 1 ? RB : 0);
    };
    // Global MFMA slot (over a slab's steps before the last) of DMA unit t of
    // n spread there, and of unit t of n spread over the last step.
    auto dma_early = [](int t, int n) constexpr { return ((2 * t + 1) * (NSTEP - 1) * NM) / (2 * n); };
    auto dma_last = [](int t, int n) constexpr { return ((2 * t + 1) * NM) / (2 * n); };

    // ---- steady state (see the header): unrolled by the ring depth, every
    // stage index a compile-time constant
    const uint32_t ldsw = __builtin_amdgcn_readfirstlane(lds0 + 1024 * wave);
    auto steady = [&](auto bc_c) -> int {
      constexpr int BC = decltype(bc_c)::value;
      constexpr int NDMA = A_PER + BC;
      constexpr int NH1 = (NDMA + 1) / 2;  // issued in the last step, after the barrier
      constexpr int NH2 = NDMA - NH1;      // issued in the next slab's earlier steps
      int s = 0;
      if (!split) return 0;
      auto unit = [&](auto stg_c, auto u_c, const i32x4& rA_, const i32x4& rB_) {
        constexpr int STG = decltype(stg_c)::value, U = decltype(u_c)::value;
        if constexpr (U < A_PER)
          dma16_off<STG * STAGE + 1024 * NW * U>(ldsw, rA_, voA[U]);
        else
          dma16_off<STG * STAGE + A_BYTES + 1024 * NW * (U - A_PER)>(ldsw, rB_, voB[U - A_PER]);
      };
      i32x4 rsAn = make_rsrc(a_panel + (kStages - 2) * a_step, a_bytes - (kStages - 2) * a_step);
      i32x4 rsBn = make_rsrc(b_panel + (kStages - 2) * b_step, b_bytes - (kStages - 2) * b_step);
      for (; s + kStages <= n_steady; s += kStages) {
        if constexpr (TIED) tied_entry();
        static_for<0, kStages>([&](auto st_c) {
          constexpr int ST = decltype(st_c)::value;         // stage of slab s + ST
          constexpr int STN = (ST + 1) % kStages;            // stage of slab s + ST + 1
          constexpr int STD = (ST + kStages - 1) % kStages;  // stage of slab s + ST + kStages - 1
          constexpr int ST2 = (ST + kStages - 2) % kStages;  // stage of slab s + ST + kStages - 2
          static_for<0, NSTEP>([&](auto q_c) {
            constexpr int Q = decltype(q_c)::value;
            constexpr bool LAST = Q == NSTEP - 1;
            if constexpr (LAST) {
              // slab s + ST + 1 has landed once at most the loads issued after
              // its last half remain; the barrier also frees stage STD
              advance_rsrc(rsAn, (uint32_t)a_step);
              advance_rsrc(rsBn, (uint32_t)b_step);
              wait_vmcnt<(kStages - 3) * NDMA>();
              block_barrier();
            }
            static_for<0, NM>([&](auto k_c) {
              constexpr int k = decltype(k_c)::value;
              constexpr int b = blk(Q, k), i = b / FN, j = b % FN;
              mma16<TIED>(acc[Q * FQ + i][j], aS[Q & 1][i], bq[j]);
              if constexpr (!LAST) {
                if constexpr ((k * FQ) % NM == 0)
                  aS[(Q + 1) & 1][k * FQ / NM] =
                      readA(st_c, std::integral_constant<int, (Q + 1) * FQ + k * FQ / NM>{});
                static_for<0, NH2>([&](auto t_c) {
                  constexpr int t = decltype(t_c)::value;
                  if constexpr (dma_early(t, NH2) == Q * NM + k)
                    unit(std::integral_constant<int, ST2>{}, std::integral_constant<int, NH1 + t>{}, rsAn, rsBn);
                });
              } else {
                if constexpr (k < FQ)
                  aS[0][k] = readA(std::integral_constant<int, STN>{}, std::integral_constant<int, k>{});
                if constexpr (k % FQ == FQ - 1)
                  bq[j] = readB(std::integral_constant<int, STN>{}, std::integral_constant<int, j>{});
                static_for<0, NH1>([&](auto t_c) {
                  constexpr int t = decltype(t_c)::value;
                  if constexpr (dma_last(t, NH1) == k)
                    unit(std::integral_constant<int, STD>{}, std::integral_constant<int, t>{}, rsAn, rsBn);
                });
              }
            });
            // (the written-out MFMAs keep their place among the memory
            // instructions by themselves)
            if constexpr (!TIED) {
              static_for<0, NM>([&](auto k_c) {
                constexpr int k = decltype(k_c)::value;
                constexpr int nr = nreads(Q, k);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);
              });
            }
          });
        });
      }
      // the second half of slab s + kStages - 2 is still due
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

    // ---- remaining slabs (and a K tail): the general loop, same steps with
    // run-time stage indices and whole-slab loads
    for (int s = s0; s < nk; ++s) {
      if constexpr (TIED) tied_entry();
      const int st = s % kStages, stn = (s + 1) % kStages;
      static_for<0, NSTEP>([&](auto q_c) {
        constexpr int Q = decltype(q_c)::value;
        constexpr bool LAST = Q == NSTEP - 1;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (LAST) {
          if (s + 1 < nk) {
            // this wave's loads of slab s + 1 are done once at most the loads
            // of the slabs issued after it remain
            const int after = (nk - 2 - s) < (kStages - 3) ? (nk - 2 - s) : (kStages - 3);
            if (after >= 3) wait_slabs(std::integral_constant<int, 3>{});
            else if (after == 2) wait_slabs(k2c);
            else if (after == 1) wait_slabs(k1c);
            else wait_slabs(k0c);
            block_barrier();
            if (s + kStages - 1 < nk) issue_slab(s + kStages - 1);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        static_for<0, NM>([&](auto k_c) {
          constexpr int k = decltype(k_c)::value;
          constexpr int b = blk(Q, k), i = b / FN, j = b % FN;
          mma16<TIED>(acc[Q * FQ + i][j], aS[Q & 1][i], bq[j]);
          if constexpr (!LAST) {
            if constexpr ((k * FQ) % NM == 0)
              aS[(Q + 1) & 1][k * FQ / NM] = readA_rt(st, (Q + 1) * FQ + k * FQ / NM);
          } else {
            // after the last slab these read a stale stage (in bounds) whose
            // values are never used
            if constexpr (k < FQ) aS[0][k] = readA_rt(stn, k);
            if constexpr (k % FQ == FQ - 1) bq[j] = readB_rt(stn, j);
          }
        });
      });
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- epilogue: each accumulator element is stored exactly once, by its
    // owner. The K loop is over, so the ring is free: each wave stages 16-row
    // strips of its sub-tile (one A block row at a time) and stores them as
    // 16-byte row chunks. Lane l holds row l16 of block row i, columns
    // 16 j + 4 lg .. + 3.
    if constexpr (TIED) settle_tied(acc);
    constexpr int ESZ = OUT_BF16 ? 2 : 4;
    constexpr int RING = kStages * STAGE;
    constexpr int SH = 16;
    constexpr int OPITCH = WTN * ESZ + 16;  // staged row pitch (bytes)
    static_assert(NW * SH * OPITCH <= RING, "a staged strip of every wave fits the ring");
    constexpr int CH = WTN * ESZ / 16;  // 16-byte chunks per staged row
    constexpr int EPC = 16 / ESZ;       // elements per chunk
    __syncthreads();  // every wave is done reading the ring
    if (glu) {
      constexpr int OPG = BN * 4 + 16;
      static_assert(WM * SH * OPG <= RING, "a block-wide fp32 strip fits the ring");
      static_assert(BN / 2 % 8 == 0 && BN / 2 / 4 <= NT, "whole output chunks per block row");
      const EpiOut eo{p.C, p.ldc, M, glu, p.bias, p.act, p.counts, p.flags};
#pragma unroll
      for (int i = 0; i < FM; ++i) {
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
      static_assert(NW * SH * OPF <= RING, "an fp32 strip of every wave fits the ring");
      static_assert(WTN / 4 <= 64, "one wave covers a staged row in 16-byte chunks");
      const uint32_t stf = lds0 + (uint32_t)(wave * SH * OPF);
      const EpiOut eo{p.C, p.ldc, M, N, p.bias, p.act, p.counts, p.flags};
#pragma unroll
      for (int i = 0; i < FM; ++i) {
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
      // the strip is private to this wave and one wave's LDS operations run
      // in order, so its reads below see its writes above
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
    // the next tile's loads reuse the ring: every wave must be done reading
    // its staged strips (the stores may still be in flight)
    wait_lgkmcnt0();
    block_barrier();
  }
}

}  // namespace tg
