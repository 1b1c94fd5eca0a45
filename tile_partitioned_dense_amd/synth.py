"""Seeded synthetic inputs, shared by the GPU tests, the benchmark and the oracle
checks.

This module draws random numbers and encodes them as bf16 bit patterns. It
holds none of the product's arithmetic, and neither the GPU library nor the
oracle imports the other through it.

Recipe (one GPU's share of the LLM projections the pages discuss; no trained
weights exist here, so every operand is synthetic):

* generator: numpy PCG64 ``default_rng(seed)`` with seed = 1000 * case + op,
  op = 1 for A, 2 for B, 3 and 4 for the integer-valued A and B;
* a fused-epilogue bias is N(0, 1) (or scaled) drawn in float64 and rounded
  once to float32;
* real-valued entries are drawn in float64, scaled in float64 and rounded
  once to bf16 (round to nearest, ties to even);
* N(0, s2) names the variance: N(0, 1/8192) has standard deviation 8192^-1/2,
  which keeps every C entry near unit variance at K = 8192;
* integer-valued entries are uniform on {-3, ..., 3}; they are exact in bf16
  and every product sum is an exact integer, so the result is unique;
* a column-major B is generated as its N x K row-major storage and used
  through the transposed view.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 to bf16 bits, once (nearest, ties to even).

    Method: narrow to fp32 with round-to-odd (truncate, then set the last bit
    if anything was dropped), then round that fp32 pattern to bf16 with
    integer nearest-even rounding. fp32 keeps 16 more bits than bf16, so the
    odd-rounded intermediate never creates a false tie: the two steps equal a
    single rounding of the fp64 value. Inputs here are finite and far from the
    fp32 subnormal and overflow ranges.
    """
    x = np.asarray(x, dtype=np.float64)
    t = x.astype(np.float32)
    back = t.astype(np.float64)
    away = (np.abs(back) > np.abs(x)).astype(np.uint32)
    inexact = (back != x).astype(np.uint32)
    u = (t.view(np.uint32) - away) | inexact     # truncate toward zero, then sticky bit
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u = u + np.uint32(0x7FFF) + lsb
    return (u >> np.uint32(16)).astype(np.uint16)


_CHUNK = 1 << 20


def draw(rows: int, cols: int, dist: str, seed: int, scale: float = 1.0) -> np.ndarray:
    """A rows x cols C-contiguous uint16 array of bf16 bit patterns.

    Values are drawn in row-major order, a million at a time (the generator's
    stream is the same as one single draw; chunking only bounds the size of
    the float64 temporaries).
    """
    if dist not in ("normal", "uniform", "int3"):
        raise ValueError(f"unknown distribution {dist!r}")
    rng = np.random.default_rng(seed)
    out = np.empty((int(rows), int(cols)), np.uint16)
    flat = out.reshape(-1)
    for s in range(0, flat.size, _CHUNK):
        n = min(_CHUNK, flat.size - s)
        if dist == "normal":
            x = rng.standard_normal(n) * float(scale)
        elif dist == "uniform":
            x = rng.uniform(-1.0, 1.0, n) * float(scale)
        else:
            x = rng.integers(-3, 4, n).astype(np.float64)
        flat[s:s + n] = f64_to_bf16_bits(x)
    return out


def draw_bias(n: int, seed: int, scale: float = 1.0) -> np.ndarray:
    """A length-n float32 bias vector: N(0, scale^2) drawn in float64 with
    ``default_rng(seed)`` and rounded once to float32."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(int(n)) * float(scale)).astype(np.float32)


@dataclass(frozen=True)
class Workload:
    name: str
    case: int              # seed family: seeds are 1000 * case + op
    M: int
    N: int
    K: int
    b_col_major: bool
    outs: tuple            # output dtypes checked: "f32" and/or "bf16"
    a_dist: str
    b_dist: str
    a_scale: float = 1.0
    b_scale: float = 1.0
    note: str = ""

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def algorithmic_bytes(self, out: str) -> int:
        """Each operand read once plus C written once."""
        esz = 4 if out == "f32" else 2
        return 2 * (self.M * self.K + self.K * self.N) + esz * self.M * self.N


_S = 1.0 / np.sqrt(8192.0)

WORKLOADS = {
    "gemm256": Workload(
        "gemm256", 1, 256, 256, 256, False, ("f32",), "uniform", "uniform",
        note="256^3, U[-1,1] entries; integer {-3..3} variant gives an exact result"),
    "square4096": Workload(
        "square4096", 2, 4096, 4096, 4096, False, ("bf16", "f32"), "normal", "normal",
        note="4096^3 square, N(0,1) entries, bf16 and fp32 outputs"),
    "qkv_shard": Workload(
        "qkv_shard", 3, 8192, 1280, 8192, False, ("f32",), "normal", "normal",
        b_scale=_S,
        note="attention QKV projection, one of 8 column shards: 8192 tokens x 8192 hidden -> 1280"),
    "mlp_gate_up_shard": Workload(
        "mlp_gate_up_shard", 4, 8192, 7168, 8192, True, ("bf16",), "normal", "normal",
        b_scale=_S,
        note="MLP gate+up projection shard, B stored column-major, bf16 output"),
    "decode": Workload(
        "decode", 5, 16, 28672, 8192, False, ("bf16",), "normal", "normal",
        b_scale=_S,
        note="decode-shaped skinny GEMM, 16 tokens, HBM-bound"),
    "decode_colB": Workload(
        "decode_colB", 6, 16, 28672, 8192, True, ("bf16",), "normal", "normal",
        b_scale=_S,
        note="the decode shape with B stored column-major (each output column's weights "
             "contiguous, the usual layout of a projection's weight matrix)"),
}

# The decode / tall-skinny sweep: decode batches of 1, 8, 32 and 64 rows against
# the same weight matrix as the decode workload (same seeds, so B is the same
# draw and A's rows are the first rows of one stream), in both B layouts, and
# the tall-skinny (4096, 256, 4096) shape.
for _m in (1, 8, 32, 64):
    WORKLOADS[f"decode_m{_m}"] = Workload(
        f"decode_m{_m}", 5, _m, 28672, 8192, False, ("bf16",), "normal", "normal", b_scale=_S,
        note=f"decode sweep: {_m} rows, B row-major")
    WORKLOADS[f"decode_colB_m{_m}"] = Workload(
        f"decode_colB_m{_m}", 6, _m, 28672, 8192, True, ("bf16",), "normal", "normal", b_scale=_S,
        note=f"decode sweep: {_m} rows, B column-major")
WORKLOADS["tall_skinny"] = Workload(
    "tall_skinny", 7, 4096, 256, 4096, False, ("bf16",), "normal", "normal", b_scale=1.0 / 64.0,
    note="tall-skinny (4096, 256, 4096), B row-major")
WORKLOADS["tall_skinny_colB"] = Workload(
    "tall_skinny_colB", 8, 4096, 256, 4096, True, ("bf16",), "normal", "normal", b_scale=1.0 / 64.0,
    note="tall-skinny (4096, 256, 4096), B column-major")
WORKLOADS["launch64"] = Workload(
    "launch64", 9, 64, 64, 64, False, ("bf16",), "uniform", "uniform",
    note="64^3: a kernel of about a microsecond, for the per-call cost")


@dataclass
class Operands:
    A: np.ndarray          # (M, K) uint16 view
    B: np.ndarray          # (K, N) uint16 view (transposed view when column-major)
    B_storage: np.ndarray  # the C-contiguous array that holds B


def operands(w: Workload, integer: bool = False, M: int | None = None,
             N: int | None = None, K: int | None = None) -> Operands:
    """Seeded operands for workload ``w`` (optionally at another shape)."""
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    if integer:
        A = draw(M, K, "int3", 1000 * w.case + 3)
        Bs = draw(N, K, "int3", 1000 * w.case + 4) if w.b_col_major else \
            draw(K, N, "int3", 1000 * w.case + 4)
    else:
        A = draw(M, K, w.a_dist, 1000 * w.case + 1, w.a_scale)
        Bs = draw(N, K, w.b_dist, 1000 * w.case + 2, w.b_scale) if w.b_col_major else \
            draw(K, N, w.b_dist, 1000 * w.case + 2, w.b_scale)
    B = Bs.T if w.b_col_major else Bs
    return Operands(A, B, Bs)


# ------------------------------------------------------------------ MX (MXFP8)
#
# MX operands are quantised from the same kind of random values: per row,
# blocks of 32 consecutive K values share a power-of-two scale 2^e (stored as
# the E8M0 byte e + 127) chosen the OCP MX way, e = floor(log2(max |x|)) - 8
# (8 being E4M3's largest exponent), and each x / 2^e is rounded to the
# nearest E4M3 value (ties to even), saturating at +-448. The integer variant
# uses the E4M3 codes of -3..3 with unit scales, so products are exact.
# The scaled-integer variant keeps those codes and draws every block's scale
# uniformly from a given range of E8M0 bytes: products are then integers
# times 2^(ea + eb), and when the exponents ea + eb of one product span at
# most S across all blocks, every partial sum of the K products is a multiple
# of 2^(min ea + eb) below 9 K 2^S of that unit. With 9 K 2^S < 2^24 each
# partial sum is exact in fp32 whatever the order of summation, so the GPU's
# result is the exact sum: the ranges used below (A in [120, 123], B in
# [131, 134], S = 6) allow K up to 29127.

MX_BLOCK = 32
_E4M3_INT_CODES = {-3: 0xC4, -2: 0xC0, -1: 0xB8, 0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44}


def f64_to_e4m3(y) -> np.ndarray:
    """Round float64 values to E4M3 codes (nearest, ties to even; saturating
    at +-448; no NaN is produced)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), 448.0)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    q = np.exp2(e - 3.0)                         # spacing of E4M3 values in [2^e, 2^(e+1))
    v = np.minimum(np.rint(a / q) * q, 448.0)    # np.rint rounds half to even
    sub = v < 2.0 ** -6
    E = np.floor(np.log2(np.where(sub, 1.0, v)))
    m = np.where(sub, 0.0, (v / np.exp2(E) - 1.0) * 8.0)
    code = np.where(sub, np.rint(v / 2.0 ** -9), (E + 7.0) * 8.0 + m).astype(np.uint8)
    return code | np.signbit(y).astype(np.uint8) << 7


_E2M1_INT_CODES = {-3: 0xD, -2: 0xC, -1: 0xA, 0: 0x0, 1: 0x2, 2: 0x4, 3: 0x5}


def f64_to_e2m1(y) -> np.ndarray:
    """Round float64 values to E2M1 codes 0..15 (nearest, ties to even;
    saturating at +-6). The spacing of E2M1 values is 0.5 below 2, 1 in
    [2, 4) and 2 in [4, 6]."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), 6.0)
    e = np.maximum(np.floor(np.log2(np.maximum(a, 1.0))), 0.0)
    q = np.exp2(e - 1.0)
    v = np.minimum(np.rint(a / q) * q, 6.0)
    idx = np.searchsorted(np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]), v)
    return (idx.astype(np.uint8) | (np.signbit(y).astype(np.uint8) << 3)).astype(np.uint8)


def pack_fp4(codes) -> np.ndarray:
    """rows x k E2M1 codes -> rows x ceil(k/2) bytes, the lower K index in the
    low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    if c.shape[1] % 2:
        c = np.pad(c, ((0, 0), (0, 1)))
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def mx_scale_stride(k: int) -> int:
    """Bytes per scale row: one per 32 K values, rounded up to a multiple of 4."""
    return (((k + MX_BLOCK - 1) // MX_BLOCK) + 3) // 4 * 4


MX_INT_SCALES_A = (120, 123)   # E8M0 bytes of A's blocks in the scaled-integer variant
MX_INT_SCALES_B = (131, 134)   # and of B's: product exponents span -3 .. 3


def draw_mx(rows: int, k: int, dist: str, seed: int, scale: float = 1.0, fmt: str = "e4m3",
            scale_codes: tuple | None = None):
    """(codes, scales): rows x k E4M3 codes (E2M1: rows x k/2 packed bytes) and
    rows x mx_scale_stride(k) E8M0 bytes (padding bytes 127). Values are drawn
    like draw() (row-major, in chunks of rows), then quantised per block of 32
    as described above (E2M1: largest exponent 2, so e = floor(log2 max) - 2).
    With dist "int3" the codes are those of -3..3; `scale_codes` = (lo, hi)
    then draws each block's scale byte uniformly from lo..hi (after all the
    codes, from the same generator), else every scale is 127 (unit)."""
    if dist not in ("normal", "uniform", "int3"):
        raise ValueError(f"unknown distribution {dist!r}")
    if fmt not in ("e4m3", "e2m1"):
        raise ValueError(f"unknown MX element format {fmt!r}")
    fp4 = fmt == "e2m1"
    emax = 2.0 if fp4 else 8.0
    encode = f64_to_e2m1 if fp4 else f64_to_e4m3
    int_codes = _E2M1_INT_CODES if fp4 else _E4M3_INT_CODES
    rng = np.random.default_rng(seed)
    ls = mx_scale_stride(k)
    codes = np.empty((rows, k), np.uint8)
    scales = np.full((rows, ls), 127, np.uint8)
    nb = (k + MX_BLOCK - 1) // MX_BLOCK
    step = max(1, (1 << 20) // max(k, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        n = (r1 - r0) * k
        if dist == "int3":
            v = rng.integers(-3, 4, n).reshape(r1 - r0, k)
            codes[r0:r1] = np.vectorize(int_codes.get, otypes=[np.uint8])(v)
            continue
        x = (rng.standard_normal(n) if dist == "normal" else rng.uniform(-1.0, 1.0, n))
        x = (x * float(scale)).reshape(r1 - r0, k)
        pad = np.zeros((r1 - r0, nb * MX_BLOCK))
        pad[:, :k] = x
        blocks = pad.reshape(r1 - r0, nb, MX_BLOCK)
        amax = np.abs(blocks).max(axis=2)
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - emax, -127.0)
        e = np.clip(e, -127.0, 127.0)
        scales[r0:r1, :nb] = (e + 127.0).astype(np.uint8)
        q = blocks / np.exp2(e)[:, :, None]
        codes[r0:r1] = encode(q).reshape(r1 - r0, nb * MX_BLOCK)[:, :k]
    if dist == "int3" and scale_codes is not None:
        lo, hi = scale_codes
        if not (0 <= lo <= hi <= 254):
            raise ValueError(f"scale bytes {scale_codes} outside 0..254")
        scales[:, :nb] = rng.integers(lo, hi + 1, (rows, nb)).astype(np.uint8)
    return (pack_fp4(codes) if fp4 else codes), scales


@dataclass(frozen=True)
class MxWorkload:
    name: str
    case: int
    M: int
    N: int
    K: int
    outs: tuple
    b_scale: float = 1.0
    note: str = ""
    fmt: str = "e4m3"

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def algorithmic_bytes(self, out: str) -> int:
        """Elements and scales read once, C written once."""
        esz = 4 if out == "f32" else 2
        ls = mx_scale_stride(self.K)
        kb = self.K // 2 if self.fmt == "e2m1" else self.K
        return (self.M + self.N) * (kb + ls) + esz * self.M * self.N


MX_WORKLOADS = {
    "mx_mlp_gate_up_shard": MxWorkload(
        "mx_mlp_gate_up_shard", 14, 8192, 7168, 8192, ("bf16",), b_scale=_S,
        note="the MLP gate+up shard in MXFP8 (weights N x K), bf16 output"),
    "mx_square4096": MxWorkload(
        "mx_square4096", 12, 4096, 4096, 4096, ("bf16",),
        note="4096^3 in MXFP8"),
    "mx_decode": MxWorkload(
        "mx_decode", 15, 16, 28672, 8192, ("bf16",), b_scale=_S,
        note="the decode shape in MXFP8, HBM-bound"),
    "mxfp4_mlp_gate_up_shard": MxWorkload(
        "mxfp4_mlp_gate_up_shard", 16, 8192, 7168, 8192, ("bf16",), b_scale=_S,
        note="the MLP gate+up shard in MXFP4 (weights N x K), bf16 output", fmt="e2m1"),
    "mxfp4_decode": MxWorkload(
        "mxfp4_decode", 17, 16, 28672, 8192, ("bf16",), b_scale=_S,
        note="the decode shape in MXFP4, HBM-bound", fmt="e2m1"),
}


@dataclass
class MxOperands:
    A: np.ndarray    # (M, K) E4M3 codes (E2M1: (M, K/2) packed)
    sA: np.ndarray   # (M, ls) E8M0
    Bt: np.ndarray   # (N, K) E4M3 codes of B's transpose
    sB: np.ndarray   # (N, ls)


def mx_operands(w: MxWorkload, integer: bool = False, M: int | None = None,
                N: int | None = None, K: int | None = None,
                varied_scales: bool = False) -> MxOperands:
    """Operands of an MX workload (optionally at another shape). integer: the
    codes of -3..3, with unit scales, or with varied_scales each block's scale
    drawn from MX_INT_SCALES_A / MX_INT_SCALES_B (seeds op 5 and 6)."""
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    if integer:
        opa, opb = (5, 6) if varied_scales else (3, 4)
        A, sA = draw_mx(M, K, "int3", 1000 * w.case + opa, fmt=w.fmt,
                        scale_codes=MX_INT_SCALES_A if varied_scales else None)
        Bt, sB = draw_mx(N, K, "int3", 1000 * w.case + opb, fmt=w.fmt,
                         scale_codes=MX_INT_SCALES_B if varied_scales else None)
        return MxOperands(A, sA, Bt, sB)
    A, sA = draw_mx(M, K, "normal", 1000 * w.case + 1, fmt=w.fmt)
    Bt, sB = draw_mx(N, K, "normal", 1000 * w.case + 2, w.b_scale, fmt=w.fmt)
    return MxOperands(A, sA, Bt, sB)
