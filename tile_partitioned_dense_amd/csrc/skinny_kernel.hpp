// skinny_kernel.hpp -- bandwidth-oriented kernel for decode-shaped GEMMs
// (M up to 64; the planner uses it for M <= 16), where streaming B from HBM
// is the whole cost: with M rows the
// arithmetic intensity is about M flops per byte of B, far below the MFMA
// ridge point, the memory-bound regime the tensor-parallel page describes
// for small GEMMs ("Implementing Tensor Parallelism Communication Overlays
// for Distributed LLM Inference in Rust", section "Performance Tradeoffs:
// Choosing the Right Chunk Size").
//
// Ownership: workgroup w owns C[0:M, 16*T*w : 16*T*(w+1)] and is its only
// writer; B's column stripe for those columns is read exactly once, by this
// workgroup. Its eight waves split K into contiguous ranges, and their
// partial sums meet in LDS along a fixed pairwise tree (wave w adds wave
// w + h for h = 4, 2, 1), the pattern of the fixed-order workgroup
// reductions in "Rust Compute Kernels" (section "Signature mapping"), so
// the per-element summation order is fixed and results are bit-identical.
//
// MFMA 16x16x32: lane l (column group nl = l % 16, k group kg = l / 16) holds
// for a 32-k block: A rows 16g + nl, k = 8kg..8kg+7 (one 16-byte load of
// the K-contiguous A), and B columns n0 + T*nl + c (c < T) for the same 8 k.
// A row-major B is read as eight k rows of T contiguous columns (coalesced:
// 16 lanes cover 32*T contiguous bytes of a row) and transposed in registers.
#pragma once

#include "common.hpp"
#include "plan.hpp"

namespace tg {

struct SkinnyArgs {
  const uint16_t* A;
  const uint16_t* B;
  void* C;
  int32_t M, N, K;
  int64_t lda, ldb, ldc;
  uint32_t* counts;  // debug instrumentation only
  int32_t flags;
  const float* bias;  // fused epilogue: N fp32 values or NULL
  int32_t act;        // fused epilogue: kAct*
  int32_t glu_half;   // SiLU(gate) * up: N / 2 (the gate's width), else 0
};

template <int T>
struct RowChunk;  // T contiguous bf16 of one row
template <>
struct RowChunk<4> {
  uint32_t w[2];
};
template <>
struct RowChunk<8> {
  uint32_t w[4];
};

template <int T>
__device__ __forceinline__ RowChunk<T> load_row_chunk(const uint16_t* src, int c, int len, bool fast) {
  RowChunk<T> r;
  if (fast || c + T <= len) {
    if constexpr (T == 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + c);
      r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(src + c);
      r.w[0] = v.x; r.w[1] = v.y;
    }
  } else {
#pragma unroll
    for (int d = 0; d < T / 2; ++d) r.w[d] = 0u;
#pragma unroll
    for (int e = 0; e < T; ++e)
      if (c + e < len) r.w[e >> 1] |= ((uint32_t)src[c + e]) << (16 * (e & 1));
  }
  return r;
}

template <int T, int NW, int MG, int U, bool BCOL, bool OUT_BF16, bool DEBUG>
__global__ __launch_bounds__(NW * 64) void skinny_gemm_kernel(SkinnyArgs p) {
  static_assert(NW == 8 || NW == 4 || NW == 2, "pairwise tree needs a power of two");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kg = lane >> 4, nl = lane & 15;
  const int M = p.M, N = p.N, K = p.K;
  // With SiLU(gate) * up a workgroup owns 8 T output columns n0 ..: lanes
  // nl < 8 read their gate columns, lanes nl >= 8 the matching up columns
  // glu + n0 + .., so both halves of an output column meet in one block.
  const int glu = p.glu_half;
  const int n0 = blockIdx.x * (glu ? 8 * T : 16 * T);      // first output column
  const int lcol = n0 + T * (glu ? (nl & 7) : nl);         // this lane's first logical column
  const int ncol = lcol + ((glu && nl >= 8) ? glu : 0);    // ... and its first column of B
  const int climit = glu ? glu : N;                        // logical columns end here
  const bool cols_full = n0 + (glu ? 8 * T : 16 * T) <= climit;

  const int nkb = (K + 31) >> 5;
  const int kb0 = (wave * nkb) / NW;
  const int kb1 = ((wave + 1) * nkb) / NW;

  floatx4 acc[MG][T];
#pragma unroll
  for (int g = 0; g < MG; ++g)
#pragma unroll
    for (int c = 0; c < T; ++c) acc[g][c] = floatx4{};

  // ---- fast path: interior column stripe, full 32-k blocks. Loads are
  // unconditional (rows of A past M are clamped to row M-1; their products
  // only reach accumulator rows that are never stored) and run DEPTH blocks
  // ahead of the MFMAs. A column-major B arrives in 64-byte pieces per column
  // and block, so it keeps more blocks in flight where the registers allow
  // (measured: 4 blocks and plain loads, whose lines then serve the
  // neighbouring piece from L2, beat 2 blocks and streaming loads by about a
  // third).
  constexpr int DEPTH = (BCOL && MG * T <= 8) ? 4 : 2;
  int kb = kb0;
  const int kb_full = kb1 < (K >> 5) ? kb1 : (K >> 5);  // end of full blocks
  if (cols_full && kb_full - kb0 >= DEPTH) {
    struct Blk {
      bf16x8 a[MG];
      RowChunk<T> rows[8];  // row-major B: 8 k rows x T columns
      bf16x8 bc[T];         // column-major B: T columns x 8 k
    };
    // per-lane element offsets (32-bit, fixed for the loop) from a uniform
    // per-block base, so each load is one SGPR base plus one VGPR offset
    uint32_t offA[MG];
#pragma unroll
    for (int g = 0; g < MG; ++g) {
      const int row = (16 * g + nl) < M ? (16 * g + nl) : (M - 1);
      offA[g] = (uint32_t)(row * p.lda + 8 * kg);
    }
    uint32_t offB[BCOL ? T : 8];
#pragma unroll
    for (int r = 0; r < (BCOL ? T : 8); ++r)
      offB[r] = BCOL ? (uint32_t)((ncol + r) * p.ldb + 8 * kg) : (uint32_t)((8 * kg + r) * p.ldb + ncol);
    auto load_blk = [&](int b, Blk& x) {
      const uint16_t* ab = p.A + b * 32;
      const uint16_t* bb = BCOL ? p.B + b * 32 : p.B + (int64_t)b * 32 * p.ldb;
#pragma unroll
      for (int g = 0; g < MG; ++g) x.a[g] = as_bf16x8(*reinterpret_cast<const uint4*>(ab + offA[g]));
      if constexpr (BCOL) {
#pragma unroll
        for (int c = 0; c < T; ++c) x.bc[c] = as_bf16x8(*reinterpret_cast<const uint4*>(bb + offB[c]));
      } else {
        // a row-major B is read exactly once in whole row segments: streaming loads
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          if constexpr (T == 8) {
            const uint4 v = load16_stream(bb + offB[r]);
            x.rows[r].w[0] = v.x; x.rows[r].w[1] = v.y; x.rows[r].w[2] = v.z; x.rows[r].w[3] = v.w;
          } else {
            const uint2 v = load8_stream(bb + offB[r]);
            x.rows[r].w[0] = v.x; x.rows[r].w[1] = v.y;
          }
        }
      }
    };
    auto compute_blk = [&](const Blk& x) {
#pragma unroll
      for (int c = 0; c < T; ++c) {
        bf16x8 bv;
        if constexpr (BCOL) {
          bv = x.bc[c];
        } else {
          uint32_t w[4];
#pragma unroll
          for (int d = 0; d < 4; ++d)
            w[d] = pack_halves(x.rows[2 * d].w[c >> 1], x.rows[2 * d + 1].w[c >> 1], (c & 1) != 0);
          bv = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
        }
#pragma unroll
        for (int g = 0; g < MG; ++g) acc[g][c] = mfma16(x.a[g], bv, acc[g][c]);
      }
    };
    Blk buf[DEPTH];
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) load_blk(kb + i, buf[i]);
    for (; kb + 2 * DEPTH <= kb_full; kb += DEPTH) {
#pragma unroll
      for (int i = 0; i < DEPTH; ++i) {
        compute_blk(buf[i]);
        load_blk(kb + DEPTH + i, buf[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) compute_blk(buf[i]);
    kb += DEPTH;
  }

  // ---- general path: the rest of this wave's blocks (edges, K tail)
  for (; kb < kb1; kb += U) {
    bf16x8 af[U][MG];
    bf16x8 bt[U][T];
    // issue every load of U blocks before the first MFMA
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = (kb + u) < kb1;
      const int kbase = (kb + u) * 32 + 8 * kg;  // this lane's 8 k values
      const bool kfull = valid && (kb + u) * 32 + 32 <= K;
#pragma unroll
      for (int g = 0; g < MG; ++g) {
        const int row = 16 * g + nl;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (valid && row < M) v = load8_masked(p.A + (int64_t)row * p.lda, kbase, K);
        af[u][g] = as_bf16x8(v);
      }
      if constexpr (BCOL) {
#pragma unroll
        for (int c = 0; c < T; ++c) {
          const int col = ncol + c;
          uint4 v = make_uint4(0, 0, 0, 0);
          if (valid && lcol + c < climit) v = load8_masked(p.B + (int64_t)col * p.ldb, kbase, K);
          bt[u][c] = as_bf16x8(v);
        }
      } else {
        RowChunk<T> rows[8];
        const bool fast = kfull && cols_full;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int gk = kbase + r;
          if (valid && gk < K && lcol < climit) {
            rows[r] = load_row_chunk<T>(p.B + (int64_t)gk * p.ldb, ncol, ncol - lcol + climit, fast);
          } else {
#pragma unroll
            for (int d = 0; d < T / 2; ++d) rows[r].w[d] = 0u;
          }
        }
        // regroup: column c of this lane = 8 k values (rows 0..7)
#pragma unroll
        for (int c = 0; c < T; ++c) {
          uint32_t w[4];
#pragma unroll
          for (int d = 0; d < 4; ++d)
            w[d] = pack_halves(rows[2 * d].w[c >> 1], rows[2 * d + 1].w[c >> 1], (c & 1) != 0);
          bt[u][c] = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int g = 0; g < MG; ++g)
#pragma unroll
        for (int c = 0; c < T; ++c) acc[g][c] = mfma16(af[u][g], bt[u][c], acc[g][c]);
  }

  // Fixed pairwise tree over the waves: for h = NW/2, ..., 1 wave w < h adds
  // wave w + h's partial sums.
  __shared__ floatx4 red[NW / 2][MG * T][64];
#pragma unroll
  for (int h = NW / 2; h >= 1; h >>= 1) {
    if (wave >= h && wave < 2 * h) {
#pragma unroll
      for (int g = 0; g < MG; ++g)
#pragma unroll
        for (int c = 0; c < T; ++c) red[wave - h][g * T + c][lane] = acc[g][c];
    }
    __syncthreads();
    if (wave < h) {
#pragma unroll
      for (int g = 0; g < MG; ++g)
#pragma unroll
        for (int c = 0; c < T; ++c) acc[g][c] += red[wave][g * T + c][lane];
    }
    __syncthreads();
  }

  if (p.bias != nullptr || p.act != kActNone) {
    // Fused epilogue: wave 0 stages the summed block as fp32 rows in LDS (the
    // tree's buffer is free again) and all waves share one rolled
    // bias / activation / store pass.
    constexpr int OPF = 16 * T * 4 + 16;
    static_assert(16 * MG * OPF <= (int)sizeof(red), "the fp32 block fits the tree's buffer");
    static_assert(16 * T / 4 <= NW * 64, "the workgroup covers a staged row in 16-byte chunks");
    const uint32_t stf = (uint32_t)(uintptr_t)&red[0][0][0];
    if (wave == 0) {
#pragma unroll
      for (int g = 0; g < MG; ++g)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int c = 0; c < T; c += 4)
            lds_store_f4(stf + (uint32_t)((16 * g + 4 * kg + v) * OPF + (T * nl + c) * 4),
                         floatx4{acc[g][c][v], acc[g][c + 1][v], acc[g][c + 2][v], acc[g][c + 3][v]});
    }
    __syncthreads();
    if (glu) {
      const EpiOut eo{p.C, p.ldc, M, glu, p.bias, p.act, p.counts, p.flags};
      store_staged_glu<OUT_BF16, DEBUG>(stf, OPF, 16 * MG, 8 * T, 16 * MG, 0, 0, n0, threadIdx.x,
                                        NW * 64, eo);
    } else {
      const EpiOut eo{p.C, p.ldc, M, N, p.bias, p.act, p.counts, p.flags};
      store_staged_fused<OUT_BF16, DEBUG>(stf, OPF, 16 * MG, 16 * T, 0, n0, threadIdx.x, NW * 64, eo);
    }
    return;
  }

  if (wave == 0) {
#pragma unroll
    for (int g = 0; g < MG; ++g) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 16 * g + 4 * kg + v;
        if (row < M) {
#pragma unroll
          for (int c = 0; c < T; ++c) {
            const int col = ncol + c;
            if (col < N) {
              const int64_t off = (int64_t)row * p.ldc + col;
              if constexpr (OUT_BF16) {
                static_cast<uint16_t*>(p.C)[off] = f32_to_bf16(acc[g][c][v]);
              } else {
                static_cast<float*>(p.C)[off] = acc[g][c][v];
              }
              if constexpr (DEBUG) {
                if (p.flags & kDbgCount) atomicAdd(p.counts + (int64_t)row * N + col, 1u);
              }
            }
          }
        }
      }
    }
  }
}

}  // namespace tg
