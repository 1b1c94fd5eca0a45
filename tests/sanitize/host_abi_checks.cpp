// host_abi_checks.cpp -- drives the host-only half of the C ABI (argument
// checks, planners, the tile map; csrc/host_abi.hpp) over ordinary, edge and
// hostile inputs. Built with g++ under the address and undefined-behaviour
// sanitizers by tests/test_host_sanitize.py, so an overflow, out-of-bounds
// access or other undefined operation in that code aborts the run; the
// driver itself checks that every returned status is a defined one and that
// every plan's tile map is a bijection onto its tile grid.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "host_abi.hpp"

namespace {

long g_calls = 0;

void require(bool ok, const char* what, long long a = 0, long long b = 0, long long c = 0) {
  if (!ok) {
    fprintf(stderr, "FAILED: %s (%lld, %lld, %lld)\n", what, a, b, c);
    exit(1);
  }
}

bool known(tile_gemm_status_t s) { return s >= TILE_GEMM_OK && s <= TILE_GEMM_ERR_EPILOGUE; }

const int64_t kDims[] = {0, 1, 2, 7, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129,
                         255, 256, 257, 1000, 1280, 4096, 7168, 8192, 28672,
                         ((int64_t)1 << 31) - 1, (int64_t)1 << 31, -1, INT64_MAX, INT64_MIN};
const int64_t kStrides[] = {0, 1, -1, 2, 16, 64, 8192, ((int64_t)1 << 31) - 16, (int64_t)1 << 31,
                            (int64_t)1 << 40, INT64_MAX, INT64_MIN};
const uintptr_t kPtrs[] = {0, 16, 0x1000, 0x100000, 0x7fff00000000ull, UINTPTR_MAX - 15};

// Every wg of an accepted plan: tiles inside the output, each owned once.
void check_map(const tile_gemm_plan_t& p, int64_t M, int64_t N) {
  if (p.tiles <= 0 || p.tiles > (1 << 20)) return;
  std::vector<char> seen((size_t)p.tiles, 0);
  for (int64_t wg = 0; wg < p.tiles; ++wg) {
    int64_t m0, n0, rows, cols;
    const tile_gemm_status_t s = tile_gemm_tile_of(&p, M, N, wg, &m0, &n0, &rows, &cols);
    ++g_calls;
    require(s == TILE_GEMM_OK, "tile_of rejected an in-range wg", wg, M, N);
    require(m0 >= 0 && n0 >= 0 && rows >= 0 && cols >= 0, "tile_of: negative", m0, n0, wg);
    require(m0 < M || M == 0, "tile_of: row outside", m0, M, wg);
    require(n0 < N, "tile_of: column outside", n0, N, wg);
    if (p.variant == TILE_GEMM_VARIANT_SKINNY) {
      const int64_t t = n0 / p.bn;
      require(t < p.tiles && !seen[(size_t)t], "skinny map: column tile twice", t, wg, N);
      seen[(size_t)t] = 1;
    } else {
      require(m0 % p.bm == 0 && n0 % p.bn == 0, "tile_of: unaligned tile", m0, n0, wg);
      const int64_t t = (m0 / p.bm) * p.tiles_n + n0 / p.bn;
      require(t < p.tiles && !seen[(size_t)t], "tile map: tile owned twice", t, wg, p.tiles);
      seen[(size_t)t] = 1;
    }
  }
  int64_t m0, n0, rows, cols;
  require(tile_gemm_tile_of(&p, M, N, p.tiles, &m0, &n0, &rows, &cols) != TILE_GEMM_OK,
          "tile_of accepted wg == tiles");
  require(tile_gemm_tile_of(&p, M, N, -1, &m0, &n0, &rows, &cols) != TILE_GEMM_OK,
          "tile_of accepted wg < 0");
  g_calls += 2;
}

void plans() {
  const int cus[] = {1, 8, 224, 256, 0, -1};
  for (int64_t M : kDims)
    for (int64_t N : kDims)
      for (int64_t K : {(int64_t)0, (int64_t)1, (int64_t)64, (int64_t)8192, (int64_t)-5,
                        ((int64_t)1 << 31)}) {
        for (int cu : cus) {
          for (int bcol = 0; bcol < 2; ++bcol) {
            tile_gemm_plan_t p;
            const tile_gemm_status_t s = tile_gemm_plan(M, N, K, bcol, cu, &p);
            ++g_calls;
            require(known(s), "plan: unknown status", M, N, K);
            if (s == TILE_GEMM_OK && M > 0 && N > 0 && M <= 65536 && N <= 65536) check_map(p, M, N);
          }
          for (int fmt = -1; fmt < 3; ++fmt) {
            tile_gemm_plan_t p;
            const tile_gemm_status_t s = tile_gemm_plan_mx(M, N, K, (tile_gemm_mx_format_t)fmt, cu, &p);
            ++g_calls;
            require(known(s), "plan_mx: unknown status", M, N, K);
            if (s == TILE_GEMM_OK && M > 0 && N > 0 && M <= 65536 && N <= 65536) check_map(p, M, N);
          }
        }
      }
  require(tile_gemm_plan(16, 16, 16, 0, 256, nullptr) == TILE_GEMM_ERR_NULL_ARG, "plan: NULL out");
  require(tile_gemm_tile_of(nullptr, 1, 1, 0, nullptr, nullptr, nullptr, nullptr) ==
              TILE_GEMM_ERR_NULL_ARG, "tile_of: NULL plan");
}

void args() {
  const int dtypes[] = {TILE_GEMM_BF16_TO_F32, TILE_GEMM_BF16_TO_BF16, 2, -1};
  const int64_t shapes[][3] = {{0, 0, 0}, {1, 1, 1}, {16, 28672, 8192}, {8192, 7168, 8192},
                               {255, 257, 33}, {((int64_t)1 << 31) - 1, 16, 16},
                               {-1, 4, 4}, {INT64_MAX, INT64_MAX, INT64_MAX}};
  for (const auto& sh : shapes)
    for (int64_t sa : kStrides)
      for (int64_t sb : kStrides)
        for (int64_t sc : kStrides)
          for (int dt : dtypes) {
            const int64_t M = sh[0], N = sh[1], K = sh[2];
            // A row-major (a_m = sa), B row-major or column-major by turns, C row-major
            const tile_gemm_strides_t st[3] = {{sa, 1, sb, 1, sc, 1},
                                               {sa, 1, 1, sb, sc, 1},
                                               {1, sa, sb, sc, 1, sc}};
            for (const auto& s : st)
              for (uintptr_t pa : kPtrs) {
                const uintptr_t pc = pa ^ 0x40000000ull;
                const tile_gemm_status_t r = tile_gemm_check_args(
                    (const void*)pa, (const void*)(pa + 0x80000000ull), (const void*)pc, M, N, K, &s,
                    (tile_gemm_dtype_t)dt);
                ++g_calls;
                require(known(r), "check_args: unknown status", M, N, K);
                require(tile_gemm_last_error_detail() != nullptr, "detail NULL");
              }
          }
  tile_gemm_strides_t s = {64, 1, 64, 1, 64, 1};
  require(tile_gemm_check_args(nullptr, nullptr, nullptr, 1, 1, 1, nullptr, TILE_GEMM_BF16_TO_F32) !=
              TILE_GEMM_OK, "check_args accepted NULL strides");
  // C inside A is refused
  require(tile_gemm_check_args((const void*)0x10000, (const void*)0x900000, (const void*)0x10000, 64,
                               64, 64, &s, TILE_GEMM_BF16_TO_F32) == TILE_GEMM_ERR_ALIAS,
          "check_args accepted C == A");
  g_calls += 2;
}

void epilogues() {
  for (int act = -2; act <= 8; ++act)
    for (uintptr_t pb : kPtrs)
      for (int64_t N : {(int64_t)0, (int64_t)16, (int64_t)24, (int64_t)7168, INT64_MAX}) {
        tile_gemm_strides_t s = {N, 1, 1, N, N, 1};
        const tile_gemm_status_t r = tile_gemm_check_epilogue(
            (const void*)0x100000, 64, N, &s, TILE_GEMM_BF16_TO_BF16, (const float*)pb,
            (tile_gemm_act_t)act);
        ++g_calls;
        require(known(r), "check_epilogue: unknown status", act, N);
      }
}

void mx() {
  const int64_t lss[] = {0, 4, 8, 256, 3, -4, ((int64_t)1 << 31), INT64_MAX};
  const int64_t shapes[][3] = {{0, 0, 0}, {16, 28672, 8192}, {8192, 7168, 8192}, {1, 64, 128},
                               {255, 257, 64}, {((int64_t)1 << 31) - 1, 64, 64}, {-1, 64, 64}};
  for (const auto& sh : shapes)
    for (int fmt = -1; fmt <= 2; ++fmt)
      for (int64_t ls : lss)
        for (int64_t sa : kStrides)
          for (int64_t sc : kStrides)
            for (int act = -1; act <= 5; ++act) {
              const tile_gemm_strides_t s = {sa, 1, 1, sa, sc, 1};
              const tile_gemm_status_t r = tile_gemm_check_mx(
                  (const void*)0x100000, (const void*)0x200000000ull, (const void*)0x400000000ull,
                  sh[0], sh[1], sh[2], &s, (const void*)0x600000000ull, (const void*)0x700000000ull,
                  ls, (tile_gemm_mx_format_t)fmt, TILE_GEMM_BF16_TO_BF16, nullptr,
                  (tile_gemm_act_t)act);
              ++g_calls;
              require(known(r), "check_mx: unknown status", sh[0], sh[1], ls);
            }
}

}  // namespace

int main() {
  for (int s = -3; s <= 12; ++s) require(tile_gemm_status_str((tile_gemm_status_t)s) != nullptr, "status_str");
  plans();
  args();
  epilogues();
  mx();
  printf("ok %ld calls\n", g_calls);
  return 0;
}
