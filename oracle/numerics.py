"""bf16 encode/decode and the acceptance rules, written for the oracle only.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Acceptance rules for a GPU result g against the oracle's fp64 C and D, with
tau = rel * D (rel = 1e-5, the tolerance stated for this product):

* fp32 output:  |g - C| <= tau; where D == 0 every term is zero and g must be 0.
* bf16 output:  RNE(C - tau) <= g <= RNE(C + tau), RNE applied directly from
  fp64. Rounding is monotone, so this is the same as "g is the bf16 rounding
  of some value within tau of C"; the 1e-5 bound cannot hold for the bf16
  value itself, whose own rounding step is up to 2^-9 relative.
* exact (integer-valued inputs): g == C numerically (fp32 output) or
  g == RNE(C) (bf16 output). Every partial sum is then an integer far below
  2^24, so any summation order gives the exact value.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) exactly to float64."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("expected uint16 bf16 bit patterns")
    u32 = b.astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def rne_bf16(x) -> np.ndarray:
    """Round float64 values to bf16 (round to nearest, ties to even).

    Rounds once, directly from fp64. bf16 keeps 8 significant bits and the
    fp32 exponent range, so a normal value a = m * 2^e (m in [0.5, 1)) is
    quantised to multiples of 2^(e-8); below 2^-126 the quantum stays at the
    smallest subnormal, 2^-133. Magnitudes that round to 2^128 or beyond
    become infinity; NaN maps to the quiet NaN 0x7FC0 with its sign.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x)
    ax = np.abs(x)
    nan = np.isnan(ax)
    ax = np.where(nan, 0.0, ax)
    _, e = np.frexp(ax)
    qexp = np.maximum(e.astype(np.int64) - 8, -133)
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.ldexp(np.rint(np.ldexp(ax, -qexp)), qexp)
        f32 = r.astype(np.float32)  # exact: r is a bf16 value, or overflows to inf
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(nan, np.uint16(0x7FC0), bits).astype(np.uint16)
    bits = bits | (sign.astype(np.uint16) << np.uint16(15))
    return bits.astype(np.uint16)


@dataclass
class CheckReport:
    ok: bool
    n: int
    n_bad: int
    max_ratio: float          # max |g - C| / D over elements with D > 0
    first_bad: tuple | None = None
    detail: str = ""
    extra: dict = field(default_factory=dict)

    def __bool__(self) -> bool:  # pragma: no cover - convenience
        return self.ok


def _first_bad(mask):
    if not mask.any():
        return None
    return tuple(int(v) for v in np.unravel_index(int(np.argmax(mask)), mask.shape))


def _ratio(g64, C, D):
    err = np.abs(g64 - C)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(D > 0, err / np.where(D > 0, D, 1.0), np.where(err > 0, np.inf, 0.0))
    r = np.where(np.isnan(g64), np.inf, r)
    return float(r.max()) if r.size else 0.0


def check_f32(g, C, D, rel: float = 1e-5) -> CheckReport:
    """fp32 output: |g - C| <= rel * D elementwise (NaN always fails)."""
    g64 = np.asarray(g, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    if g64.shape != C.shape or C.shape != D.shape:
        raise ValueError(f"shape mismatch {g64.shape} {C.shape} {D.shape}")
    tau = rel * D
    good = np.abs(g64 - C) <= tau
    bad = ~good
    nb = int(bad.sum())
    return CheckReport(nb == 0, int(g64.size), nb, _ratio(g64, C, D), _first_bad(bad),
                       f"fp32 |g-C| <= {rel:g}*D")


def check_bf16(gbits, C, D, rel: float = 1e-5) -> CheckReport:
    """bf16 output: RNE(C - tau) <= g <= RNE(C + tau), tau = rel * D."""
    gbits = np.asarray(gbits)
    C = np.asarray(C, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    if gbits.shape != C.shape or C.shape != D.shape:
        raise ValueError("shape mismatch")
    tau = rel * D
    lo = bf16_to_f64(rne_bf16(C - tau))
    hi = bf16_to_f64(rne_bf16(C + tau))
    g = bf16_to_f64(gbits)
    good = (lo <= g) & (g <= hi)
    bad = ~good
    nb = int(bad.sum())
    return CheckReport(nb == 0, int(g.size), nb, _ratio(g, C, D), _first_bad(bad),
                       f"bf16 RNE(C -/+ {rel:g}*D) bracket")


def check_exact(g, C, out_bf16: bool) -> CheckReport:
    """Integer-valued inputs: numeric equality with C (fp32) or RNE(C) (bf16)."""
    C = np.asarray(C, dtype=np.float64)
    if out_bf16:
        g64 = bf16_to_f64(np.asarray(g))
        want = bf16_to_f64(rne_bf16(C))
    else:
        g64 = np.asarray(g, dtype=np.float64)
        want = C
    if g64.shape != want.shape:
        raise ValueError("shape mismatch")
    bad = ~(g64 == want)
    nb = int(bad.sum())
    return CheckReport(nb == 0, int(g64.size), nb,
                       float(np.abs(g64 - want).max()) if g64.size else 0.0,
                       _first_bad(bad), "exact")
