/*
 * tile_gemm.h -- C ABI of the tile-partitioned dense GEMM for AMD Instinct
 * MI355X (gfx950).
 *
 * Operation: C = A . B with bf16 inputs, fp32 accumulation and an fp32 or
 * bf16 output. This is the dense product the pages measure at
 * M = N = K = 8192 ("GPU speed, without leaving Rust's safety model",
 * section "Safety without a visible tax"), built on the partition discipline
 * of the same page (sections "Ownership crosses the launch boundary" and
 * "The useful boundary"): the output is split into disjoint tiles before
 * launch, each tile is exclusively owned by one workgroup, the only writer of
 * it, and A and B are shared read-only views.
 *
 * Numerics: every output element is the sum of its K products accumulated in
 * fp32 in one fixed ascending-k order that depends only on the shape and the
 * B layout, never on the output type, timing or run. There is no split-K and
 * no atomic accumulation, so results are bit-identical from run to run, and
 * a bf16 output is the round-to-nearest-even of the fp32 result of the same
 * shape.
 *
 * Threading: a handle's plan state is read-only after tile_gemm_create, so
 * concurrent tile_gemm_run calls on different streams may share it (the
 * optional plan log below is guarded by a lock inside the handle).
 */
#ifndef TILE_GEMM_H
#define TILE_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TILE_GEMM_ABI_VERSION 1

/* Opaque, host-side handle. */
typedef struct tile_gemm_handle* tile_gemm_t;

typedef enum {
  TILE_GEMM_OK = 0,
  TILE_GEMM_ERR_NULL_ARG = 1,   /* a required pointer is NULL */
  TILE_GEMM_ERR_BAD_SHAPE = 2,  /* M, N or K negative, or too large for 32-bit tile indices */
  TILE_GEMM_ERR_BAD_STRIDE = 3, /* a layout other than the accepted ones below */
  TILE_GEMM_ERR_MISALIGNED = 4, /* base pointer or leading dimension not 16-byte aligned */
  TILE_GEMM_ERR_ALIAS = 5,      /* C's bytes overlap A's or B's */
  TILE_GEMM_ERR_DTYPE = 6,      /* unknown tile_gemm_dtype_t */
  TILE_GEMM_ERR_DEVICE = 7,     /* no such device, not gfx950, or not the current device */
  TILE_GEMM_ERR_HIP = 8,        /* the HIP runtime refused a call or a launch */
  TILE_GEMM_ERR_EPILOGUE = 9    /* unknown activation in a fused epilogue */
} tile_gemm_status_t;

/* Input is always bf16 with fp32 accumulation; the enum picks the output. */
typedef enum {
  TILE_GEMM_BF16_TO_F32 = 0,
  TILE_GEMM_BF16_TO_BF16 = 1
} tile_gemm_dtype_t;

/*
 * Strides in elements (not bytes). Element (i, k) of A is A[i*a_m + k*a_k],
 * element (k, j) of B is B[k*b_k + j*b_n], element (i, j) of C is
 * C[i*c_m + j*c_n]. Accepted layouts (anything else is
 * TILE_GEMM_ERR_BAD_STRIDE):
 *   A: a_k == 1 and a_m >= K                       (row-major)
 *   B: b_n == 1 and b_k >= N                       (row-major), or
 *      b_k == 1 and b_n >= K                       (column-major)
 *   C: c_n == 1 and c_m >= N                       (row-major)
 */
typedef struct {
  int64_t a_m, a_k;
  int64_t b_k, b_n;
  int64_t c_m, c_n;
} tile_gemm_strides_t;

/*
 * One-time set-up for `device` (a HIP device ordinal): checks that it is a
 * gfx950 and records its compute-unit count, which the planner uses. Allocates
 * no device memory. On success *out holds a new handle; on failure *out is
 * set to NULL (when out is not NULL).
 * Errors: TILE_GEMM_ERR_NULL_ARG (out == NULL), TILE_GEMM_ERR_DEVICE.
 *
 * Environment, read here once: TILE_GEMM_LOG set to anything but "" or "0"
 * makes every run entry point print the plan it launches (variant,
 * configuration, tile, K step, threads, tiles, grid) to stderr, once per
 * distinct call shape (the first 64 shapes; every call after that).
 *
 * Source: the split between a once-only preparation and cheap recording of
 * work ("Rust Compute Kernels", section "Quick example": prepare compiles or
 * hits the cache once, record only appends), and an operation built once and
 * then driven synchronously, chained or replayed from a graph ("GPU speed,
 * without leaving Rust's safety model", section "Build once, choose how to
 * execute"). The handle is what is prepared once; every run reuses it.
 */
tile_gemm_status_t tile_gemm_create(tile_gemm_t* out, int device);

/*
 * Source: the output partitioned into disjoint owned tiles with the inputs as
 * shared read-only views, and a launcher that holds its operands while the
 * work is in flight ("GPU speed, without leaving Rust's safety model", section
 * "Ownership crosses the launch boundary"); capture into a graph limited to
 * operations that allocate nothing (same page, section "Why scoped graph
 * capture helps borrowing"). The signature is C = A . B with shape, strides,
 * output type and stream.
 *
 * Enqueue C := A . B on `stream` (a hipStream_t; NULL means the default
 * stream) and return without waiting. A and B are device pointers to bf16
 * data, C a device pointer to fp32 or bf16 data per `dtype`; all three must be
 * 16-byte aligned, and each leading dimension (a_m, the non-unit B stride,
 * c_m) times the element size must be a multiple of 16 bytes.
 *
 * Ownership: A and B are borrowed read-only and C exclusively until the
 * stream reaches this work; the caller must not free, write (or, for C, read)
 * them before then. The library neither frees nor retains caller memory.
 * tile_gemm_run allocates nothing and never synchronises, so it may be
 * captured into a HIP graph.
 *
 * Shapes: M = 0 or N = 0 is a successful no-op (pointers are not checked);
 * K = 0 writes zeros to C (A and B are not read: they may be NULL and their
 * strides are not checked). M, N and K must be below 2^31, and A and B must
 * each span less than 4 GiB (TILE_GEMM_ERR_BAD_SHAPE otherwise); the leading
 * dimensions a_m, the non-unit B stride and c_m must be below 2^31 elements
 * (TILE_GEMM_ERR_BAD_STRIDE otherwise), and every byte span is computed with
 * overflow checks, so no stride can wrap an extent past the 4 GiB and overlap
 * checks.
 *
 * Errors are returned before anything is enqueued and leave C untouched:
 * NULL_ARG, BAD_SHAPE, BAD_STRIDE, MISALIGNED, ALIAS, DTYPE, DEVICE (the
 * calling thread's current device is not the handle's). A launch the
 * runtime rejects returns TILE_GEMM_ERR_HIP. Faults during execution surface
 * at the caller's next synchronisation of the stream.
 */
tile_gemm_status_t tile_gemm_run(tile_gemm_t h, const void* A, const void* B, void* C,
                                 int64_t M, int64_t N, int64_t K,
                                 const tile_gemm_strides_t* strides,
                                 tile_gemm_dtype_t dtype, void* stream);

/*
 * Fused epilogue: the store applies act(C + bias) to each element of the owned
 * tile before writing it, in the spirit of the epilogue fusion the TorchInductor
 * page describes ("TorchInductor ganha suporte a GEMMs de alta performance com
 * CuteDSL": a bias addition or an activation folded into the GEMM's store;
 * element-wise operations and ReLU, sigmoid, tanh in its roadmap paragraph).
 * SiLU is x * sigmoid(x).
 *
 * TILE_GEMM_ACT_SWIGLU is the gated step that follows a merged gate+up
 * projection (the column-sharded MLP of the tensor-parallel page,
 * "Implementing Tensor Parallelism Communication Overlays for Distributed LLM
 * Inference in Rust"): B's first N/2 columns are the gate, its last N/2 the
 * up projection, and the output is the M x N/2 matrix
 * silu(x[i][j]) * x[i][j + N/2], x = A.B + bias. Each output element is
 * owned and written once by the workgroup that computes both of its product
 * columns, so the single-writer rule holds for the narrower output too.
 */
typedef enum {
  TILE_GEMM_ACT_NONE = 0,
  TILE_GEMM_ACT_RELU = 1,     /* max(x, 0) */
  TILE_GEMM_ACT_SIGMOID = 2,  /* 1 / (1 + e^-x) */
  TILE_GEMM_ACT_TANH = 3,     /* tanh x */
  TILE_GEMM_ACT_SILU = 4,     /* x / (1 + e^-x) */
  TILE_GEMM_ACT_SWIGLU = 5    /* silu(gate) * up over the two halves of B's columns */
} tile_gemm_act_t;

/*
 * As tile_gemm_run, storing C[i][j] = act(sum_k A[i][k] B[k][j] + bias[j]).
 * The sum is accumulated exactly as in tile_gemm_run (same kernels, tiles and
 * K order); bias[j] is added and act evaluated in fp32, then the value is
 * stored as dtype says (a bf16 output is the round-to-nearest-even of that
 * fp32 value). `bias` is a device pointer to N fp32 values, read-only, 16-byte
 * aligned, not overlapping C; NULL means no bias. With K = 0 the result is
 * act(bias[j]) (act(0) without a bias).
 * With TILE_GEMM_ACT_SWIGLU, N counts B's columns (gate and up; a multiple of
 * 16, else TILE_GEMM_ERR_BAD_SHAPE), C is M x N/2 (c_m >= N/2) and bias, if
 * given, holds N values (gate biases, then up biases).
 * Errors: as tile_gemm_run, plus TILE_GEMM_ERR_EPILOGUE (unknown act),
 * TILE_GEMM_ERR_MISALIGNED (bias) and TILE_GEMM_ERR_ALIAS (bias overlaps C).
 */
tile_gemm_status_t tile_gemm_run_epilogue(tile_gemm_t h, const void* A, const void* B, void* C,
                                          int64_t M, int64_t N, int64_t K,
                                          const tile_gemm_strides_t* strides,
                                          tile_gemm_dtype_t dtype, const float* bias,
                                          tile_gemm_act_t act, void* stream);

/*
 * Microscaled FP8 / FP4 product (MXFP8, MXFP4), the low-precision GEMMs the
 * TorchInductor page measures beside bf16 ("TorchInductor ganha suporte a GEMMs de alta
 * performance com CuteDSL", its MXFP8 benchmark paragraph). The format is
 * read as OCP Microscaling (MX) v1.0: elements are FP8 E4M3 bytes (or FP4
 * E2M1 nibbles, see TILE_GEMM_MX_E2M1), and every 32 consecutive elements of a
 * row along K share one E8M0 scale byte (value 2^(e - 127); 255 is NaN).
 *
 *   C[i][j] = sum_k (sa[i][k/32] * a[i][k]) * (sb[j][k/32] * b[j][k])
 *
 * For E4M3, A is M x K bytes, row-major (strides a_m >= K, a_k = 1, in bytes). B is
 * given as its N x K transpose, K-contiguous (b_k = 1, b_n >= K, in bytes):
 * the layout in which weight matrices are usually stored. a_scale is M rows
 * and b_scale N rows of `scale_stride` bytes (a multiple of 4, >= K/32), the
 * scale of element k of a row at byte k/32. K must be a multiple of 64 for
 * E4M3 and of 128 for E2M1 (TILE_GEMM_ERR_BAD_SHAPE otherwise). C, dtype, bias and act (not
 * TILE_GEMM_ACT_SWIGLU) are as for tile_gemm_run_epilogue; accumulation is
 * fp32 in ascending K, one owner per output tile, each element written once.
 * Outputs of up to 64 rows run a kernel that streams B in 256-byte pieces of
 * K per row (plan bk = 256; 512 for few-column outputs of up to 32 rows);
 * larger ones the tile kernel (bk = 64).
 * A, B 16-byte aligned with 16-byte leading dimensions; scales 4-byte aligned.
 * Leading dimensions and scale_stride below 2^31 bytes, and the scale rows
 * (up to 256 past the last row of A or B) times scale_stride below 2 GiB
 * (TILE_GEMM_ERR_BAD_STRIDE or TILE_GEMM_ERR_BAD_SHAPE otherwise).
 * All inputs are borrowed read-only until the stream reaches the work; C may
 * overlap none of them. Enqueue-only, allocates nothing.
 */
typedef enum {
  TILE_GEMM_MX_E4M3 = 0, /* MXFP8: E4M3 elements, E8M0 scales per 32 */
  TILE_GEMM_MX_E2M1 = 1  /* MXFP4: E2M1 elements, two per byte (the lower K index in
                            the low nibble), E8M0 scales per 32; rows of A and B are
                            K/2 bytes, strides in bytes; K a multiple of 128 */
} tile_gemm_mx_format_t;

tile_gemm_status_t tile_gemm_run_mx(tile_gemm_t h, const void* A, const void* B, void* C,
                                    int64_t M, int64_t N, int64_t K,
                                    const tile_gemm_strides_t* strides, const void* a_scale,
                                    const void* b_scale, int64_t scale_stride,
                                    tile_gemm_mx_format_t fmt, tile_gemm_dtype_t dtype,
                                    const float* bias, tile_gemm_act_t act, void* stream);

/*
 * Release a handle (host memory only). NULL is accepted and returns OK.
 * Source: the counterpart of the one-time preparation ("Rust Compute
 * Kernels", section "Quick example"); it touches no device memory, since the
 * handle owns none, and caller buffers are never freed by the library (the
 * launcher returns borrowed operands in their ownership form: "GPU speed,
 * without leaving Rust's safety model", section "Ownership crosses the launch
 * boundary").
 */
tile_gemm_status_t tile_gemm_destroy(tile_gemm_t h);

/*
 * Static text for a status code; never NULL. Source: argument errors are
 * reported when work is recorded, before anything is bound or launched, and
 * name what was wrong ("Rust Compute Kernels", section "Shape contracts").
 * Unknown codes map to a fixed "unknown status" text.
 */
const char* tile_gemm_status_str(tile_gemm_status_t s);

/*
 * Text naming the argument (and axis) behind the last non-OK status returned
 * on the calling thread, in the spirit of the pages' record-time shape
 * contracts, which name the parameter, axis, expected and actual extent
 * ("Rust Compute Kernels", section "Shape contracts"). Empty when none.
 */
const char* tile_gemm_last_error_detail(void);

/* ---------------------------------------------------------------------- */
/* Host-only introspection. No device is touched; these work without a GPU. */

/*
 * The argument checks tile_gemm_run performs before any launch, in the same
 * order and with the same results (except the device check, which needs a
 * handle).
 */
tile_gemm_status_t tile_gemm_check_args(const void* A, const void* B, const void* C,
                                        int64_t M, int64_t N, int64_t K,
                                        const tile_gemm_strides_t* strides,
                                        tile_gemm_dtype_t dtype);

/*
 * The checks tile_gemm_run_epilogue adds for its epilogue arguments (after
 * those of tile_gemm_check_args, which for TILE_GEMM_ACT_SWIGLU it applies
 * with C's width N/2), with the same results.
 */
tile_gemm_status_t tile_gemm_check_epilogue(const void* C, int64_t M, int64_t N,
                                            const tile_gemm_strides_t* strides,
                                            tile_gemm_dtype_t dtype, const float* bias,
                                            tile_gemm_act_t act);

/* The checks tile_gemm_run_mx performs before any launch, with the same results. */
tile_gemm_status_t tile_gemm_check_mx(const void* A, const void* B, const void* C, int64_t M,
                                      int64_t N, int64_t K, const tile_gemm_strides_t* strides,
                                      const void* a_scale, const void* b_scale,
                                      int64_t scale_stride, tile_gemm_mx_format_t fmt,
                                      tile_gemm_dtype_t dtype, const float* bias,
                                      tile_gemm_act_t act);

/* Kernel variants the planner chooses between. */
typedef enum {
  TILE_GEMM_VARIANT_NONE = 0,   /* M == 0 or N == 0: nothing to launch */
  TILE_GEMM_VARIANT_TILE = 1,   /* LDS-staged MFMA tile kernel */
  TILE_GEMM_VARIANT_SKINNY = 2, /* HBM-streaming kernel, chosen for M <= 16 */
  TILE_GEMM_VARIANT_MX = 3      /* MXFP8 tile kernel (tile_gemm_run_mx) */
} tile_gemm_variant_t;

/*
 * The launch plan for a shape: a pure function of (M, N, K, B layout,
 * compute-unit count). The output type never changes it.
 *   tile kernel:   C is cut into tiles = tiles_m*tiles_n tiles of bm x bn.
 *                  When they fit in one round on the compute units every
 *                  workgroup owns one (grid = tiles); otherwise grid is about
 *                  tiles / ceil(tiles / cu_count) (a multiple of 8) and
 *                  workgroup w owns tiles w, w + grid, w + 2 grid, ..., each
 *                  whole, with its own K loop and store.
 *                  With a column-major B, an even K and M <= 64 the tile
 *                  variant runs the stream configurations (32 x 64 tiles
 *                  with bk = 256 up to 32 rows, 64 x 128 with bk = 128
 *                  above, 64 x 64 when N is small: K moves 512 or 256 bytes
 *                  per row at a time, for a weight stream bound by HBM).
 *   skinny kernel: each workgroup owns rows [0, M) x bn columns; the waves of
 *                  one workgroup split K and combine their partial sums in a
 *                  fixed order; grid = tiles = tiles_n, tiles_m = 1.
 */
typedef struct {
  int32_t variant;      /* tile_gemm_variant_t */
  int32_t config;       /* index into the compiled configuration table */
  int32_t bm, bn, bk;   /* owned tile rows, columns; K slab per step */
  int32_t threads;      /* threads per workgroup */
  int32_t lds_bytes;    /* static LDS per workgroup */
  int32_t tiles_m, tiles_n;
  int32_t group_m;      /* tile rows per raster group */
  int32_t xcds;         /* dispatch remap width (XCD count), 1 = identity */
  int32_t k_split;      /* skinny kernel: waves sharing K inside one workgroup */
  int64_t grid;         /* workgroups launched */
  int64_t tiles;        /* owned tiles (each owned by exactly one workgroup) */
} tile_gemm_plan_t;

/* b_col_major: 0 for row-major B, 1 for column-major B. cu_count > 0. */
tile_gemm_status_t tile_gemm_plan(int64_t M, int64_t N, int64_t K, int b_col_major,
                                  int cu_count, tile_gemm_plan_t* out);

/* The plan of tile_gemm_run_mx for a shape and element format (variant
 * TILE_GEMM_VARIANT_MX; the configurations rank differently for E4M3 and
 * E2M1). An unknown fmt is TILE_GEMM_ERR_DTYPE. */
tile_gemm_status_t tile_gemm_plan_mx(int64_t M, int64_t N, int64_t K, tile_gemm_mx_format_t fmt,
                                     int cu_count, tile_gemm_plan_t* out);

/*
 * Tile number `wg` (0 <= wg < plan->tiles) under `plan`: rows [m0, m0 + rows)
 * and columns [n0, n0 + cols) of C, clipped to M x N. Workgroup w of the
 * launch owns tile numbers w, w + grid, ... This is the very function the
 * kernels run, compiled for the host, so tests can check that the map is a
 * bijection onto the tiles and that the tiles exactly cover C.
 */
tile_gemm_status_t tile_gemm_tile_of(const tile_gemm_plan_t* plan, int64_t M, int64_t N,
                                     int64_t wg, int64_t* m0, int64_t* n0,
                                     int64_t* rows, int64_t* cols);

/* ---------------------------------------------------------------------- */
/* Test instrumentation. Same kernels, extra bookkeeping; not for production. */

enum {
  TILE_GEMM_DEBUG_COUNT_WRITES = 1, /* each element store also adds 1 to counts[i*N + j] */
  TILE_GEMM_DEBUG_COLLIDE = 2       /* negative control: workgroup 1 takes workgroup 0's tile */
};
/* Run a given compiled configuration instead of the planner's choice, so tests
 * can cover every configuration at small sizes. A forced skinny configuration
 * needs M <= its row capacity (16 * row groups); a forced stream
 * configuration a column-major B and an even K (else TILE_GEMM_ERR_BAD_SHAPE).
 * Forced configurations and
 * grids run the production kernel instances; only TILE_GEMM_DEBUG_COUNT_WRITES
 * and TILE_GEMM_DEBUG_COLLIDE select the instrumented ones. */
#define TILE_GEMM_DEBUG_FORCE_TILE(c) ((((c) + 1) & 0xff) << 8)
#define TILE_GEMM_DEBUG_FORCE_SKINNY(c) ((((c) + 1) & 0xff) << 16)
/* Launch g workgroups (1 <= g <= 126, at most the tile count) for the tile
 * kernel instead of the planner's grid, so each takes several tiles; or, with
 * TILE_GEMM_DEBUG_ONE_TILE_PER_WG, one workgroup per tile. */
#define TILE_GEMM_DEBUG_FORCE_GRID(g) (((g) & 0x7f) << 24)
/* Raster group height g (1 <= g <= 63 tile rows; clipped to the tile rows)
 * for the tile kernel's owned-tile map instead of the planner's, so the
 * effect of the tile order on cache traffic can be measured. Any height keeps
 * the map a bijection. */
#define TILE_GEMM_DEBUG_GROUP_M(g) (((g) & 0x3f) << 2)
#define TILE_GEMM_DEBUG_ONE_TILE_PER_WG (0x7f << 24)

/*
 * As tile_gemm_run, with instrumentation. `counts` is a device array of M*N
 * uint32 (row-major, N columns) that the caller zeroes; it is required when
 * TILE_GEMM_DEBUG_COUNT_WRITES is set and ignored otherwise. Every element of
 * a correct run has count 1; TILE_GEMM_DEBUG_COLLIDE deliberately breaks the
 * tile map (two workgroups own one tile, another tile has no owner) so tests
 * can show that their checks catch a partition error. The collision needs at
 * least two tiles and applies to the tile kernel only. Unknown flag bits or an
 * unknown forced configuration return TILE_GEMM_ERR_BAD_SHAPE. `bias` and `act`
 * are the fused epilogue of tile_gemm_run_epilogue (NULL and
 * TILE_GEMM_ACT_NONE for the plain product), so tests can run it on every
 * configuration.
 */
tile_gemm_status_t tile_gemm_run_debug(tile_gemm_t h, const void* A, const void* B, void* C,
                                       int64_t M, int64_t N, int64_t K,
                                       const tile_gemm_strides_t* strides,
                                       tile_gemm_dtype_t dtype, void* stream,
                                       uint32_t* counts, int flags, const float* bias,
                                       tile_gemm_act_t act);

/*
 * As tile_gemm_run_mx, with the instrumentation of tile_gemm_run_debug
 * (TILE_GEMM_DEBUG_FORCE_TILE(c) forces MX configuration c).
 */
tile_gemm_status_t tile_gemm_run_mx_debug(tile_gemm_t h, const void* A, const void* B, void* C,
                                          int64_t M, int64_t N, int64_t K,
                                          const tile_gemm_strides_t* strides,
                                          const void* a_scale, const void* b_scale,
                                          int64_t scale_stride, tile_gemm_mx_format_t fmt,
                                          tile_gemm_dtype_t dtype, const float* bias,
                                          tile_gemm_act_t act, void* stream, uint32_t* counts,
                                          int flags);

#ifdef __cplusplus
}
#endif

#endif /* TILE_GEMM_H */
