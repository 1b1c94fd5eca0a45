"""CPU checks of the MX input generator (synth.draw_mx): its E4M3 rounding
against torch's float8_e4m3fn conversion, and the OCP block-scale rule."""

import numpy as np
import pytest

from tile_partitioned_dense_amd import synth
from oracle import mx


def test_e4m3_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000) * 60, rng.standard_normal(20000) * 0.01,
                        [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 3 * 2.0 ** -10, 1.5 * 2.0 ** -9,
                         1.0625 * 2.0 ** -6, 9.5, 10.5, 0.5 + 2.0 ** -5]])
    x = np.clip(x, -448.0, 448.0)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(synth.f64_to_e4m3(x), ref)


def test_draw_mx_block_scales():
    A, s = synth.draw_mx(8, 100, "normal", 3)
    assert A.shape == (8, 100) and s.shape == (8, synth.mx_scale_stride(100)) == (8, 4)
    v = mx.e4m3_to_f64(A)
    for r in range(8):
        for b in range(4):
            blk = np.abs(v[r, 32 * b:32 * b + 32])
            if blk.size:
                # the largest element of a block sits in [256, 448] (the scale
                # is floor(log2 amax) - 8, so amax / 2^e lies in [256, 512))
                assert 256.0 <= blk.max() <= 448.0


def test_draw_mx_integer_variant_is_exact_small_integers():
    A, s = synth.draw_mx(4, 64, "int3", 5)
    v = mx.e4m3_to_f64(A)
    assert set(np.unique(v)).issubset({-3.0, -2.0, -1.0, 0.0, 1.0, 2.0, 3.0})
    assert (s == 127).all()


def _nearest_e2m1(y):
    """Brute force: the nearest of the 8 magnitudes, ties to the even code."""
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    out = []
    for v in np.asarray(y, dtype=np.float64):
        a = min(abs(v), 6.0)
        d = np.abs(mags - a)
        best = np.nonzero(d == d.min())[0]
        idx = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        out.append(idx | (8 if np.signbit(v) else 0))
    return np.array(out, np.uint8)


def test_e2m1_rounding_brute_force():
    rng = np.random.default_rng(1)
    y = np.concatenate([rng.uniform(-7, 7, 4000), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, 6.5,
                                                   -0.0, 0.0, 0.24, 2.49]])
    assert np.array_equal(synth.f64_to_e2m1(y), _nearest_e2m1(y))


def test_draw_mx_fp4_packing_and_scales():
    A, s = synth.draw_mx(6, 96, "normal", 4, fmt="e2m1")
    assert A.shape == (6, 48) and s.shape == (6, 4)
    v = mx.mx_decode(A, s, 96, "e2m1") / np.exp2(s[:, np.arange(96) // 32].astype(float) - 127)
    for r in range(6):
        for b in range(3):
            blk = np.abs(v[r, 32 * b:32 * b + 32])
            assert 4.0 <= blk.max() <= 6.0     # amax / 2^e in [4, 8), saturating at 6
    Ai, si = synth.draw_mx(3, 64, "int3", 5, fmt="e2m1")
    vi = mx.mx_decode(Ai, si, 64, "e2m1")
    assert set(np.unique(vi)).issubset({-3.0, -2.0, -1.0, 0.0, 1.0, 2.0, 3.0})


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_draw_mx_scaled_integer_variant(fmt):
    """Integer codes with per-block scales drawn from the stated ranges: the
    scales vary from block to block and row to row, stay inside the range,
    and the exactness condition 9 K 2^S < 2^24 holds for the ranges the tests
    use at K = 8192 (S: spread of the product exponents)."""
    k = 1024
    A, sA = synth.draw_mx(40, k, "int3", 11, fmt=fmt, scale_codes=synth.MX_INT_SCALES_A)
    B, sB = synth.draw_mx(40, k, "int3", 12, fmt=fmt, scale_codes=synth.MX_INT_SCALES_B)
    nb = k // 32
    for s, (lo, hi) in ((sA, synth.MX_INT_SCALES_A), (sB, synth.MX_INT_SCALES_B)):
        blocks = s[:, :nb]
        assert blocks.min() == lo and blocks.max() == hi
        assert len(np.unique(blocks[0])) == hi - lo + 1        # varies along K
        assert len(np.unique(blocks[:, 0])) > 1                # and across rows
        assert (s[:, nb:] == 127).all()                        # padding untouched
    dec = mx.e2m1_to_f64(mx.unpack_fp4(A, k)) if fmt == "e2m1" else mx.e4m3_to_f64(A)
    assert set(np.unique(dec)).issubset({-3.0, -2.0, -1.0, 0.0, 1.0, 2.0, 3.0})
    lo = synth.MX_INT_SCALES_A[0] + synth.MX_INT_SCALES_B[0]
    hi = synth.MX_INT_SCALES_A[1] + synth.MX_INT_SCALES_B[1]
    assert 9 * 8192 * 2 ** (hi - lo) < 2 ** 24


def test_scaled_integer_product_is_exact_in_fp32_any_order():
    """The reason the exact GPU test may demand equality: with these scales,
    summing the K scaled products in fp32 in ascending, descending or a random
    order gives the fp64 sum exactly (a check of the claim on the CPU)."""
    k = 4096
    A, sA = synth.draw_mx(3, k, "int3", 21, scale_codes=synth.MX_INT_SCALES_A)
    B, sB = synth.draw_mx(3, k, "int3", 22, scale_codes=synth.MX_INT_SCALES_B)
    a = mx.mx_decode(A, sA, k)
    b = mx.mx_decode(B, sB, k)
    rng = np.random.default_rng(0)
    for i in range(3):
        p = (a[i] * b[i]).astype(np.float64)
        exact = float(p.sum())
        for order in (np.arange(k), np.arange(k)[::-1], rng.permutation(k)):
            acc = np.float32(0.0)
            for v in p[order].astype(np.float32):
                acc = np.float32(acc + v)
            assert float(acc) == exact
