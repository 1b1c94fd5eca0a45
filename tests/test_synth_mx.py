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
