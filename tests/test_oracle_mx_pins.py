"""Pins for the oracle's microscaled (MX) product (CPU only).

Each pin ties oracle/mx.py to something other than its own formulas: the
hand-derived E4M3 and E2M1 tables in tests/golden (from the OCP MX field
layouts), torch's own float8_e4m3fn decoding of all 256 codes, closed forms
of the E8M0 scale, exact rational brute force of the scaled product, the
integer-valued case against an int64 product, the block-scale structure
(changing one block's scale changes exactly that block's contribution), and
planted mistakes that each pin set must catch.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import mx

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _table(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        if val == "nan":
            v = math.nan
        elif val == "-0":
            v = -0.0
        elif val.startswith("2^"):
            v = 2.0 ** int(val[2:])
        else:
            v = float(val)
        rows.append((int(code, 16), v))
    return rows


def _same(a, b):
    if math.isnan(b):
        return math.isnan(a)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


def pin_e4m3_golden(dec):
    for code, want in _table("e4m3_cases.txt"):
        got = float(dec(np.array([code], np.uint8))[0])
        assert _same(got, want), (hex(code), got, want)


def pin_e4m3_against_torch(dec):
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = dec(codes)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    assert np.array_equal(got[~both_nan], ref[~both_nan])


def pin_e2m1_golden(dec):
    for code, want in _table("e2m1_cases.txt"):
        got = float(dec(np.array([code], np.uint8))[0])
        assert _same(got, want), (hex(code), got, want)


def pin_e8m0(dec):
    v = dec(np.array([127, 128, 126, 0, 254, 255], np.uint8))
    assert v[:5].tolist() == [1.0, 2.0, 0.5, 2.0 ** -127, 2.0 ** 127]
    assert math.isnan(v[5])


def test_e4m3_decode_golden():
    pin_e4m3_golden(mx.e4m3_to_f64)


def test_e4m3_decode_matches_torch_for_every_code():
    pin_e4m3_against_torch(mx.e4m3_to_f64)


def test_e2m1_decode_golden():
    pin_e2m1_golden(mx.e2m1_to_f64)


def test_e8m0_decode():
    pin_e8m0(mx.e8m0_to_f64)


def test_fp4_unpack_low_nibble_first():
    packed = np.array([[0x21, 0x7f]], np.uint8)
    assert mx.unpack_fp4(packed, 4).tolist() == [[1, 2, 15, 7]]
    assert mx.unpack_fp4(packed, 3).tolist() == [[1, 2, 15]]


# ------------------------------------------------------------ the product

def _rand_mx(rng, rows, k, fmt):
    if fmt == "e4m3":
        e = rng.integers(0, 256, (rows, k)).astype(np.uint8)
        e[(e & 0x7f) == 0x7f] = 0x38                      # no NaN codes
    else:
        e = rng.integers(0, 256, (rows, (k + 1) // 2)).astype(np.uint8)
    s = rng.integers(120, 135, (rows, (k + 31) // 32)).astype(np.uint8)
    return e, s


def _frac_value(code, scale, fmt):
    v = (mx.e4m3_to_f64 if fmt == "e4m3" else mx.e2m1_to_f64)(np.array([code], np.uint8))[0]
    return Fraction(float(v)) * Fraction(2) ** (int(scale) - 127)


def pin_brute_force(gemm):
    rng = np.random.default_rng(1)
    for fmt in ("e4m3", "e2m1"):
        M, N, K = 3, 4, 70                                 # three blocks, the last partial
        A, sA = _rand_mx(rng, M, K, fmt)
        Bt, sB = _rand_mx(rng, N, K, fmt)
        C, D = gemm(A, sA, Bt, sB, K, fmt)
        ac = A if fmt == "e4m3" else mx.unpack_fp4(A, K)
        bc = Bt if fmt == "e4m3" else mx.unpack_fp4(Bt, K)
        for i in range(M):
            for j in range(N):
                exact = sum(_frac_value(ac[i, k], sA[i, k // 32], fmt)
                            * _frac_value(bc[j, k], sB[j, k // 32], fmt) for k in range(K))
                mag = sum(abs(_frac_value(ac[i, k], sA[i, k // 32], fmt)
                              * _frac_value(bc[j, k], sB[j, k // 32], fmt)) for k in range(K))
                assert abs(Fraction(C[i, j]) - exact) <= K * Fraction(2) ** -53 * mag, (fmt, i, j)
                assert abs(Fraction(D[i, j]) - mag) <= K * Fraction(2) ** -53 * mag


def pin_integer_exact(gemm):
    """Codes of small integers with unit scales: the product is the integer
    matrix product, exactly."""
    rng = np.random.default_rng(2)
    ints = {1: 0x38, 2: 0x40, 3: 0x44, -1: 0xb8, -2: 0xc0, -3: 0xc4, 0: 0x00}
    keys = np.array(sorted(ints))
    M, N, K = 5, 6, 96
    ia = rng.choice(keys, (M, K))
    ib = rng.choice(keys, (N, K))
    A = np.vectorize(ints.get)(ia).astype(np.uint8)
    Bt = np.vectorize(ints.get)(ib).astype(np.uint8)
    one = np.full((M, K // 32), 127, np.uint8)
    C, _ = gemm(A, one, Bt, np.full((N, K // 32), 127, np.uint8), K, "e4m3")
    assert np.array_equal(C, (ia.astype(np.int64) @ ib.T.astype(np.int64)).astype(np.float64))


def pin_block_scales(gemm):
    """Raising one block's scale exponent by 3 multiplies exactly that block's
    32 products by 8: the difference is 7 times that block's partial sum."""
    rng = np.random.default_rng(3)
    M, N, K = 4, 5, 128
    A, sA = _rand_mx(rng, M, K, "e4m3")
    Bt, sB = _rand_mx(rng, N, K, "e4m3")
    C0, _ = gemm(A, sA, Bt, sB, K, "e4m3")
    sA2 = sA.copy()
    sA2[1, 2] += 3
    C1, _ = gemm(A, sA2, Bt, sB, K, "e4m3")
    # rows other than 1 unchanged
    assert np.array_equal(np.delete(C1, 1, 0), np.delete(C0, 1, 0))
    A3 = A.copy()
    keep = np.zeros(K, bool)
    keep[64:96] = True
    A3[:, ~keep] = 0
    part, _ = gemm(A3, sA, Bt, sB, K, "e4m3")
    assert np.allclose(C1[1] - C0[1], 7.0 * part[1], rtol=1e-12, atol=1e-300)


def pin_layout(gemm):
    """A one-hot A picks one row of Bt: C[i, j] = sA * sB * b[j, k0]."""
    rng = np.random.default_rng(4)
    M, N, K = 2, 3, 64
    _, sA = _rand_mx(rng, M, K, "e4m3")
    Bt, sB = _rand_mx(rng, N, K, "e4m3")
    A = np.zeros((M, K), np.uint8)
    A[0, 37] = 0x38                                     # a[0][37] = 1
    A[1, 5] = 0x40                                      # a[1][5] = 2
    C, _ = gemm(A, sA, Bt, sB, K, "e4m3")
    b = mx.e4m3_to_f64(Bt)
    sa = 2.0 ** (sA.astype(np.float64) - 127)
    sb = 2.0 ** (sB.astype(np.float64) - 127)
    assert np.array_equal(C[0], sa[0, 1] * sb[:, 1] * b[:, 37])
    assert np.array_equal(C[1], 2.0 * sa[1, 0] * sb[:, 0] * b[:, 5])


PINS = [pin_brute_force, pin_integer_exact, pin_block_scales, pin_layout]


@pytest.mark.parametrize("pin", PINS)
def test_mx_gemm_pins(pin):
    pin(mx.mx_gemm)


def test_mx_gemm_at_matches_the_full_product():
    rng = np.random.default_rng(5)
    M, N, K = 6, 7, 160
    A, sA = _rand_mx(rng, M, K, "e4m3")
    Bt, sB = _rand_mx(rng, N, K, "e4m3")
    C, D = mx.mx_gemm(A, sA, Bt, sB, K)
    ii, jj = np.array([0, 5, 3]), np.array([6, 0, 2])
    c, d = mx.mx_gemm_at(A, sA, Bt, sB, K, ii, jj)
    bound = K * 2.0 ** -53 * D[ii, jj]
    assert np.all(np.abs(c - C[ii, jj]) <= bound)
    assert np.all(np.abs(d - D[ii, jj]) <= bound)


# ------------------------------------------------------- planted mistakes

def _dec_bias8(codes):
    b = np.asarray(codes, np.uint8).astype(np.int64)
    v = mx.e4m3_to_f64(codes)
    return np.where(((b >> 3) & 0xF) == 0, v, v / 2.0)       # exponent bias 8


def _dec_no_subnormal(codes):
    b = np.asarray(codes, np.uint8).astype(np.int64)
    v = mx.e4m3_to_f64(codes)
    e, m = (b >> 3) & 0xF, (b & 7).astype(np.float64)
    return np.where(e == 0, np.where(b >> 7, -1.0, 1.0) * (1 + m / 8) * 2.0 ** -7, v)


def _dec_nan_as_480(codes):
    v = mx.e4m3_to_f64(codes)
    return np.where(np.isnan(v), 480.0, v)


@pytest.mark.parametrize("bad", [_dec_bias8, _dec_no_subnormal, _dec_nan_as_480])
def test_planted_decode_mistakes_are_caught(bad):
    caught = 0
    for pin in (pin_e4m3_golden, pin_e4m3_against_torch):
        try:
            pin(bad)
        except AssertionError:
            caught += 1
    assert caught >= 1


def _gemm_with(decode_scale=None, block=None, transpose_b=False):
    def gemm(A, sA, Bt, sB, k, fmt="e4m3", want_d=True):
        def dec(e, s):
            v = mx.e4m3_to_f64(np.asarray(e)[:, :k]) if fmt == "e4m3" else \
                mx.e2m1_to_f64(mx.unpack_fp4(e, k))
            sc = (decode_scale or mx.e8m0_to_f64)(np.asarray(s))
            blk = np.minimum(np.arange(k) // (block or 32), sc.shape[1] - 1)
            return v * sc[:, blk]
        a, b = dec(A, sA), dec(Bt, sB)
        C = a @ (b if transpose_b and b.shape[0] == b.shape[1] else b.T)
        return C, np.abs(a) @ np.abs(b).T
    return gemm


PLANTED = {
    "scale bias 128": _gemm_with(decode_scale=lambda s: 2.0 ** (np.asarray(s, float) - 128)),
    "block of 16": _gemm_with(block=16),
    "block of 64": _gemm_with(block=64),
    "scale ignored": _gemm_with(decode_scale=lambda s: np.ones(np.asarray(s).shape)),
}


@pytest.mark.parametrize("name", sorted(PLANTED))
def test_planted_product_mistakes_are_caught(name):
    bad = PLANTED[name]
    caught = 0
    for pin in PINS:
        try:
            pin(bad)
        except AssertionError:
            caught += 1
    assert caught >= 1, name


def test_the_unmodified_product_passes_through_the_same_driver():
    good = _gemm_with()
    for pin in PINS:
        pin(good)


# ------------------------------------------------------------- tolerance

def test_mx_bound_closed_form():
    """One run of 8 with products 1, 2^-14 and zeros: T = 7 * 2^-13 plus the
    fp32 term; integer-valued products keep every bit (T far below 1)."""
    A = np.zeros((1, 64), np.uint8)
    Bt = np.zeros((1, 64), np.uint8)
    A[0, 0] = 0x38                                     # 1
    Bt[0, 0] = 0x38
    one = np.full((1, 2), 127, np.uint8)
    T = mx.mx_bound(A, one, Bt, one, 64)
    assert T[0, 0] == 7 * 2.0 ** -13 + 10 * 2.0 ** -24 * 1.0
    # two runs: maxima 448 * 1 (E = 8) and 1 (E = 0)
    A[0, 8] = 0x7e
    Bt[0, 8] = 0x38
    T = mx.mx_bound(A, one, Bt, one, 64)
    assert T[0, 0] == 7 * (2.0 ** -13 + 2.0 ** -5) + 10 * 2.0 ** -24 * 449.0


def test_check_mx_accepts_within_and_rejects_beyond():
    rng = np.random.default_rng(9)
    M, N, K = 5, 6, 128
    A, sA = _rand_mx(rng, M, K, "e4m3")
    Bt, sB = _rand_mx(rng, N, K, "e4m3")
    C, D = mx.mx_gemm(A, sA, Bt, sB, K)
    T = mx.mx_bound(A, sA, Bt, sB, K)
    assert np.all(T > 0)
    assert mx.check_mx(C.astype(np.float32), C, T).ok
    off = C.copy()
    off[1, 2] += 2 * T[1, 2]
    rep = mx.check_mx(off, C, T)
    assert not rep.ok and rep.first_bad == (1, 2)
    from oracle import rne_bf16
    assert mx.check_mx(rne_bf16(C), C, T, out_bf16=True).ok
    t = mx.mx_bound_at(A, sA, Bt, sB, K, [1, 4], [2, 0])
    assert np.array_equal(t, T[[1, 4], [2, 0]])
