/*
 * gemm_oracle.c -- plain, slow CPU reference for the dense product C = A.B
 * over bf16 inputs.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this library. The GPU library never
 * links, includes or calls anything here, and nothing here is shared with it:
 * this file has its own bf16 decode and its own loops.
 *
 * What it computes (the plain definition of the operation the pages build
 * their tile programs around: "GPU speed, without leaving Rust's safety
 * model", section "Safety without a visible tax", dense GEMM at
 * M = N = K = 8192):
 *
 *     C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j]
 *     D[i][j] = sum_{k=0}^{K-1} |A[i][k]| * |B[k][j]|     (tolerance scale)
 *
 * Arithmetic: every bf16 input is decoded exactly to fp64 (bits << 16 is the
 * fp32 pattern, fp32 -> fp64 is exact). A product of two bf16 values has at
 * most 16 significant bits, so it is exact in fp64; each partial sum is then
 * rounded once in fp64, in ascending k order for every element. The result is
 * within K * 2^-53 * D[i][j] of the exact rational sum; with integer-valued
 * inputs whose partial sums stay below 2^53 it is exact.
 *
 * Loop order is i-k-j (rows in parallel with OpenMP, one thread per row), so
 * every element still accumulates its own terms in ascending k; parallelism
 * never changes a sum.
 *
 * Layout: element (r, c) of a matrix lives at base[r * rs + c * cs] (strides
 * in elements), which covers row-major A and both row- and column-major B.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 is the upper half of an IEEE binary32 pattern. */
static double oracle_bf16_to_f64(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Decode a strided bf16 matrix into a dense row-major fp64 array. */
static void oracle_decode(const uint16_t* src, int64_t rows, int64_t cols,
                          int64_t rs, int64_t cs, double* dst) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c)
      dst[r * cols + c] = oracle_bf16_to_f64(src[r * rs + c * cs]);
}

int oracle_abi_version(void) { return 1; }

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Full product. C (and D unless NULL) are dense row-major M x N fp64 arrays.
 * A is M x K with strides (a_m, a_k); B is K x N with strides (b_k, b_n).
 * nthreads <= 0 means the OpenMP default. Returns 0, or -1 on a bad argument
 * or a failed allocation.
 */
int oracle_gemm_f64(const uint16_t* A, int64_t a_m, int64_t a_k,
                    const uint16_t* B, int64_t b_k, int64_t b_n,
                    int64_t M, int64_t N, int64_t K,
                    double* C, double* D, int nthreads) {
  if (M < 0 || N < 0 || K < 0 || !C) return -1;
  if (M == 0 || N == 0) return 0;
  double* B64 = NULL;
  if (K > 0) {
    if (!A || !B) return -1;
    B64 = (double*)malloc((size_t)K * (size_t)N * sizeof(double));
    if (!B64) return -1;
    oracle_decode(B, K, N, b_k, b_n, B64);
  }
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int64_t i = 0; i < M; ++i) {
    double* c = C + i * N;
    double* d = D ? D + i * N : NULL;
    for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
    if (d)
      for (int64_t j = 0; j < N; ++j) d[j] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double a = oracle_bf16_to_f64(A[i * a_m + k * a_k]);
      const double* b = B64 + k * N;
      for (int64_t j = 0; j < N; ++j) c[j] += a * b[j];
      if (d) {
        const double aa = fabs(a);
        for (int64_t j = 0; j < N; ++j) d[j] += aa * fabs(b[j]);
      }
    }
  }
  free(B64);
  return 0;
}

/*
 * Selected elements only: for each pair (ii[t], jj[t]) the same ascending-k
 * sum as oracle_gemm_f64, computed one element at a time, so sampled checks
 * of full-size products need no full-size work. d may be NULL.
 */
int oracle_gemm_f64_at(const uint16_t* A, int64_t a_m, int64_t a_k,
                       const uint16_t* B, int64_t b_k, int64_t b_n,
                       int64_t K, const int64_t* ii, const int64_t* jj,
                       int64_t count, double* c, double* d, int nthreads) {
  if (K < 0 || count < 0 || !ii || !jj || !c) return -1;
  if (K > 0 && (!A || !B)) return -1;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
  for (int64_t t = 0; t < count; ++t) {
    const int64_t i = ii[t], j = jj[t];
    double s = 0.0, sa = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double a = oracle_bf16_to_f64(A[i * a_m + k * a_k]);
      const double b = oracle_bf16_to_f64(B[k * b_k + j * b_n]);
      s += a * b;
      sa += fabs(a) * fabs(b);
    }
    c[t] = s;
    if (d) d[t] = sa;
  }
  return 0;
}
