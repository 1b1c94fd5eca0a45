"""Pins for the oracle's fused epilogue, act(C + bias) (CPU only).

Each pin ties oracle.epilogue to something other than its own formulas:
closed-form values of the activations at points where they are rational,
identities between independently computed functions (numpy's tanh against the
oracle's sigmoid; the odd part of silu), a scalar brute-force loop with
Python's math module, the acceptance rule on perturbed results, and planted
mistakes that each pin set must catch.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import fused_epilogue as ep

LN3, LN2 = math.log(3.0), math.log(2.0)


def pin_closed_forms(act_f64):
    assert act_f64([-1.5, 0.0, 2.0], "relu").tolist() == [0.0, 0.0, 2.0]
    assert act_f64([0.0], "sigmoid")[0] == 0.5
    assert abs(act_f64([LN3], "sigmoid")[0] - 0.75) < 1e-15          # 1 / (1 + 1/3)
    assert abs(act_f64([-LN3], "sigmoid")[0] - 0.25) < 1e-15
    assert act_f64([0.0], "tanh")[0] == 0.0
    assert abs(act_f64([LN2], "tanh")[0] - 0.6) < 1e-15               # (2 - 1/2) / (2 + 1/2)
    assert act_f64([0.0], "silu")[0] == 0.0
    assert abs(act_f64([LN3], "silu")[0] - 0.75 * LN3) < 1e-15
    assert act_f64([-2.5, 3.0], "none").tolist() == [-2.5, 3.0]


def pin_identities(act_f64):
    x = np.linspace(-30, 30, 2401)
    s = act_f64(x, "sigmoid")
    assert np.allclose(act_f64(-x, "sigmoid"), 1.0 - s, rtol=0, atol=1e-15)
    # tanh (numpy) against the oracle's sigmoid: tanh x = 2 sigmoid(2x) - 1
    assert np.allclose(act_f64(x, "tanh"), 2.0 * act_f64(2.0 * x, "sigmoid") - 1.0, rtol=0, atol=1e-14)
    # silu(x) - silu(-x) = x (sigmoid(x) + sigmoid(-x) = 1)
    assert np.allclose(act_f64(x, "silu") - act_f64(-x, "silu"), x, rtol=0, atol=1e-13)
    # relu(x) - relu(-x) = x
    assert np.array_equal(act_f64(x, "relu") - act_f64(-x, "relu"), x)
    # saturation without NaN
    big = np.array([-800.0, 800.0])
    assert act_f64(big, "sigmoid").tolist() == [0.0, 1.0]
    assert act_f64(big, "tanh").tolist() == [-1.0, 1.0]
    assert act_f64(big, "silu").tolist() == [0.0, 800.0]


def _brute(C, bias, act):
    ref = {"none": lambda v: v, "relu": lambda v: v if v > 0 else 0.0,
           "sigmoid": lambda v: 1.0 / (1.0 + math.exp(-v)), "tanh": math.tanh,
           "silu": lambda v: v / (1.0 + math.exp(-v))}[act]
    M, N = C.shape
    out = np.empty((M, N))
    for i in range(M):
        for j in range(N):
            out[i, j] = ref(float(C[i, j]) + (float(bias[j]) if bias is not None else 0.0))
    return out


def pin_brute_force(epilogue):
    rng = np.random.default_rng(7)
    C = rng.normal(size=(5, 7)) * 3
    b = rng.normal(size=7).astype(np.float32)
    for act in oracle.ACTS:
        for bias in (None, b):
            got = epilogue(C, bias, act)
            want = _brute(C, bias, act)
            assert np.allclose(got, want, rtol=1e-14, atol=1e-300), act


@pytest.mark.parametrize("pin", [pin_closed_forms, pin_identities])
def test_activation_pins(pin):
    pin(oracle.act_f64)


def test_bias_and_activation_brute_force():
    pin_brute_force(oracle.epilogue)


def test_bias_is_per_column():
    C = np.zeros((3, 4))
    out = oracle.epilogue(C, np.array([1.0, -2.0, 3.0, 0.5], np.float32), "none")
    assert np.array_equal(out, np.tile([1.0, -2.0, 3.0, 0.5], (3, 1)))


@pytest.mark.parametrize("act", oracle.ACTS)
def test_check_epilogue_accepts_the_reference_and_rejects_twice_the_bound(act):
    rng = np.random.default_rng(3)
    C = rng.normal(size=(16, 24)) * 4
    D = np.abs(C) * 10 + 1.0
    b = rng.normal(size=24).astype(np.float32)
    y = oracle.epilogue(C, b, act)
    t = oracle.epilogue_bound(C, D, b, act)
    assert oracle.check_epilogue(y.astype(np.float32), C, D, b, act).ok
    assert oracle.check_epilogue(oracle.rne_bf16(y), C, D, b, act, out_bf16=True).ok
    off = y.copy()
    off[2, 5] += 2.0 * t[2, 5]
    rep = oracle.check_epilogue(off, C, D, b, act)
    assert not rep.ok and rep.first_bad == (2, 5)
    nan = y.copy()
    nan[0, 0] = np.nan
    assert not oracle.check_epilogue(nan, C, D, b, act).ok


MUTANTS = {
    "sigmoid sign": lambda x, a: (1.0 / (1.0 + np.exp(np.asarray(x, float))) if a == "sigmoid"
                                  else ep.act_f64(x, a)),
    "silu without x": lambda x, a: (1.0 / (1.0 + np.exp(-np.asarray(x, float))) if a == "silu"
                                    else ep.act_f64(x, a)),
    "relu as abs": lambda x, a: (np.abs(np.asarray(x, float)) if a == "relu" else ep.act_f64(x, a)),
    "tanh as sigmoid": lambda x, a: (ep.act_f64(x, "sigmoid") if a == "tanh" else ep.act_f64(x, a)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_activation_mistakes_are_caught(name):
    bad = MUTANTS[name]
    caught = 0
    for pin in (pin_closed_forms, pin_identities):
        try:
            pin(bad)
        except AssertionError:
            caught += 1
    assert caught >= 1, name


def test_planted_bias_mistake_is_caught():
    def row_bias(C, bias=None, act="none"):      # bias indexed by row instead of column
        C = np.asarray(C, float)
        x = C if bias is None else C + np.resize(np.asarray(bias, float), C.shape[0])[:, None]
        return ep.act_f64(x, act)
    with pytest.raises(AssertionError):
        pin_brute_force(row_bias)


# ------------------------------------------------------ SiLU(gate) * up

def pin_swiglu_closed_forms(swiglu):
    # gate ln 3, up 2: silu(ln 3) = (3/4) ln 3, times 2
    C = np.array([[LN3, 0.0, -LN3, 2.0, 5.0, 4.0]])
    y = swiglu(C)
    assert y.shape == (1, 3)
    assert abs(y[0, 0] - 1.5 * LN3) < 1e-15
    assert y[0, 1] == 0.0                                   # silu(0) = 0
    assert abs(y[0, 2] - 4.0 * (-0.25 * LN3)) < 1e-15       # silu(-ln 3) = -(1/4) ln 3
    # the bias (length N) shifts both halves: C = 0, gate bias ln 3, up bias 2
    b = np.array([LN3, 0.0, 2.0, -1.0])
    y = swiglu(np.zeros((2, 4)), b)
    assert np.allclose(y, [[1.5 * LN3, 0.0]] * 2, rtol=0, atol=1e-15)


def pin_swiglu_reductions(swiglu):
    rng = np.random.default_rng(5)
    g = rng.normal(size=(4, 6)) * 4
    # up = 1: plain silu of the gate (the oracle's silu is pinned above)
    assert np.allclose(swiglu(np.hstack([g, np.ones_like(g)])), oracle.act_f64(g, "silu"),
                       rtol=1e-15, atol=0)
    # up = 0: zero; gate large: silu(g) ~ g, so the product ~ g * up
    assert np.array_equal(swiglu(np.hstack([g, np.zeros_like(g)])), np.zeros_like(g))
    u = rng.normal(size=(4, 6))
    big = np.full_like(g, 60.0)
    assert np.allclose(swiglu(np.hstack([big, u])), 60.0 * u, rtol=1e-15, atol=0)


def _swiglu_brute(C, bias):
    M, N = C.shape
    h = N // 2
    out = np.empty((M, h))
    for i in range(M):
        for j in range(h):
            gv = float(C[i, j]) + (float(bias[j]) if bias is not None else 0.0)
            uv = float(C[i, j + h]) + (float(bias[j + h]) if bias is not None else 0.0)
            out[i, j] = gv / (1.0 + math.exp(-gv)) * uv
    return out


def pin_swiglu_brute_force(swiglu):
    rng = np.random.default_rng(8)
    C = rng.normal(size=(5, 10)) * 3
    b = rng.normal(size=10).astype(np.float32)
    for bias in (None, b):
        assert np.allclose(swiglu(C, bias), _swiglu_brute(C, bias), rtol=1e-14, atol=1e-300)


@pytest.mark.parametrize("pin", [pin_swiglu_closed_forms, pin_swiglu_reductions,
                                 pin_swiglu_brute_force])
def test_swiglu_pins(pin):
    pin(oracle.swiglu)


def test_swiglu_rejects_odd_width():
    with pytest.raises(ValueError):
        oracle.swiglu(np.zeros((2, 5)))


def test_check_swiglu_accepts_the_reference_and_rejects_twice_the_bound():
    rng = np.random.default_rng(4)
    C = rng.normal(size=(12, 32)) * 3
    D = np.abs(C) * 10 + 1.0
    b = rng.normal(size=32).astype(np.float32)
    y = oracle.swiglu(C, b)
    t = oracle.swiglu_bound(C, D, b)
    assert oracle.check_swiglu(y.astype(np.float32), C, D, b).ok
    assert oracle.check_swiglu(oracle.rne_bf16(y), C, D, b, out_bf16=True).ok
    off = y.copy()
    off[3, 7] -= 2.0 * t[3, 7]
    rep = oracle.check_swiglu(off, C, D, b)
    assert not rep.ok and rep.first_bad == (3, 7)
    # an error the size of the gate's accumulation bound, propagated through
    # the product, is inside; ten times it is not
    Cg = C.copy()
    Cg[:, :16] += 1e-5 * D[:, :16]
    assert oracle.check_swiglu(oracle.swiglu(Cg, b), C, D, b).ok
    Cg[:, :16] += 9e-5 * D[:, :16]
    assert not oracle.check_swiglu(oracle.swiglu(Cg, b), C, D, b).ok


def _sw_mutant(kind):
    def f(C, bias=None):
        C = np.asarray(C, float)
        h = C.shape[1] // 2
        x = C if bias is None else C + np.asarray(bias, float)[None, :]
        g, u = x[:, :h], x[:, h:]
        if kind == "halves swapped":
            g, u = u, g
        if kind == "bias on gate only" and bias is not None:
            u = C[:, h:]
        if kind == "sigmoid gate":
            return oracle.act_f64(g, "sigmoid") * u
        if kind == "up squared":
            return oracle.act_f64(g, "silu") * u * u
        if kind == "interleaved halves":
            g, u = x[:, 0::2], x[:, 1::2]
        return oracle.act_f64(g, "silu") * u
    return f


@pytest.mark.parametrize("kind", ["halves swapped", "bias on gate only", "sigmoid gate",
                                  "up squared", "interleaved halves"])
def test_planted_swiglu_mistakes_are_caught(kind):
    bad = _sw_mutant(kind)
    caught = 0
    for pin in (pin_swiglu_closed_forms, pin_swiglu_reductions, pin_swiglu_brute_force):
        try:
            pin(bad)
        except AssertionError:
            caught += 1
    assert caught >= 1, kind


# ------------------------------------------------- the acceptance bounds' values
#
# epilogue_bound's value, worked out by hand for single elements (the rule in
# oracle/fused_epilogue.py: L (tau + 2^-22 |x|) + 2^-20 |y| + 2^-126 with
# tau = 1e-5 D, x = C + bias, y = act(x), L = 1, 1/4, 1, 1.1 for none/relu/tanh,
# sigmoid, silu). Each expected value below is a number, not a call of the
# bound: a bound ten times too loose (or tight), a wrong Lipschitz constant or
# a missing term fails here.

EPS22, EPS20, TINY = 2.0 ** -22, 2.0 ** -20, 2.0 ** -126

BOUND_CASES = [
    # act, C, D, bias, expected t
    ("none", 2.0, 100.0, None, 1e-3 + 2 * EPS22 + 2 * EPS20 + TINY),
    ("sigmoid", 0.0, 8.0, None, 0.25 * 8e-5 + 0.5 * EPS20 + TINY),
    ("relu", -3.0, 1000.0, 0.5, 1e-2 + 2.5 * EPS22 + TINY),
    ("relu", 3.0, 1000.0, 0.5, 1e-2 + 3.5 * EPS22 + 3.5 * EPS20 + TINY),
    ("tanh", LN2, 50.0, None, 5e-4 + LN2 * EPS22 + 0.6 * EPS20 + TINY),
    ("silu", LN3, 0.0, None, 1.1 * LN3 * EPS22 + 0.75 * LN3 * EPS20 + TINY),
    ("silu", 0.0, 0.0, None, TINY),
]


def pin_epilogue_bound(bound):
    for act, c, d, b, want in BOUND_CASES:
        bias = None if b is None else np.array([b], np.float32)
        t = float(bound(np.array([[c]]), np.array([[d]]), bias, act)[0, 0])
        assert abs(t - want) <= 1e-12 * want, (act, c, d, b, t, want)


# swiglu_bound, by hand: gate g, up u, e_g = 1e-5 D_g + 2^-22 |g|, e_u likewise,
# t = 1.1 |u| e_g + |silu g| e_u + 1.1 e_g e_u + 2^-20 |silu(g) u| + 2^-126.
def _sw_want(g, u, dg, du):
    eg, eu = 1e-5 * dg + EPS22 * abs(g), 1e-5 * du + EPS22 * abs(u)
    sg = g / (1.0 + math.exp(-g))
    return 1.1 * abs(u) * eg + abs(sg) * eu + 1.1 * eg * eu + EPS20 * abs(sg * u) + TINY


SW_CASES = [(LN3, 2.0, 100.0, 10.0), (0.0, 5.0, 1000.0, 1.0), (-LN3, -4.0, 0.0, 0.0)]


def pin_swiglu_bound(bound):
    for g, u, dg, du in SW_CASES:
        t = float(bound(np.array([[g, u]]), np.array([[dg, du]]))[0, 0])
        # closed form of the first case, fully by hand: silu(ln 3) = 0.75 ln 3
        want = _sw_want(g, u, dg, du)
        assert abs(t - want) <= 1e-12 * want, (g, u, dg, du, t, want)
    e = 1e-3 + EPS22 * LN3
    f = 1e-4 + 2 * EPS22
    hand = 1.1 * 2 * e + 0.75 * LN3 * f + 1.1 * e * f + EPS20 * 1.5 * LN3 + TINY
    t0 = float(bound(np.array([[LN3, 2.0]]), np.array([[100.0, 10.0]]))[0, 0])
    assert abs(t0 - hand) <= 1e-12 * hand


def test_epilogue_bound_values():
    pin_epilogue_bound(oracle.epilogue_bound)


def test_swiglu_bound_values():
    pin_swiglu_bound(oracle.swiglu_bound)


def test_epilogue_bound_is_what_fp32_arithmetic_needs():
    """Not too tight: the product accumulated in fp32 (error well inside
    1e-5 D), the bias added in fp32 and the activation evaluated in fp32 land
    inside the bound; and with the accumulation error set to its full
    allowance 1e-5 D the result still lands inside."""
    rng = np.random.default_rng(11)
    K = 512
    A = rng.normal(size=(8, K))
    B = rng.normal(size=(K, 12)) / np.sqrt(K)
    C = A @ B
    D = np.abs(A) @ np.abs(B)
    b = rng.normal(size=12).astype(np.float32)
    acc = np.zeros((8, 12), np.float32)
    for k in range(K):
        acc = (acc + (A[:, k:k + 1].astype(np.float32) * B[k:k + 1].astype(np.float32))).astype(np.float32)
    for act in oracle.ACTS:
        x32 = (acc + b[None, :]).astype(np.float32)
        x64 = x32.astype(np.float64)
        y32 = oracle.act_f64(x64, act).astype(np.float32)     # fp32 rounding of the activation
        Ce = C + 1e-5 * D * 0.999                              # worst allowed accumulation error
        y_worst = oracle.act_f64(Ce + b.astype(np.float64)[None, :], act)
        for g in (y32, y_worst):
            rep = oracle.check_epilogue(np.asarray(g, np.float64), C, D, b, act)
            assert rep.ok, (act, rep)


BOUND_MUTANTS = {
    "ten times looser": lambda C, D, bias=None, act="none", rel=1e-5, tau=None:
        10.0 * ep.epilogue_bound(C, D, bias, act, rel, tau),
    "ten times tighter": lambda C, D, bias=None, act="none", rel=1e-5, tau=None:
        0.1 * ep.epilogue_bound(C, D, bias, act, rel, tau),
    "sigmoid slope 1": lambda C, D, bias=None, act="none", rel=1e-5, tau=None:
        ep.epilogue_bound(C, D, bias, "none" if act == "sigmoid" else act, rel, tau),
    "no bias-add rounding": lambda C, D, bias=None, act="none", rel=1e-5, tau=None:
        ep.epilogue_bound(C, D, bias, act, rel, tau)
        - ep.LIPSCHITZ[act] * 2.0 ** -22 * np.abs(np.asarray(C, float)
                                                  + (0 if bias is None else np.asarray(bias, float))),
}


@pytest.mark.parametrize("name", sorted(BOUND_MUTANTS))
def test_planted_bound_mistakes_are_caught(name):
    with pytest.raises(AssertionError):
        pin_epilogue_bound(BOUND_MUTANTS[name])


@pytest.mark.parametrize("scale", [10.0, 0.1])
def test_planted_swiglu_bound_mistakes_are_caught(scale):
    with pytest.raises(AssertionError):
        pin_swiglu_bound(lambda C, D, bias=None, rel=1e-5: scale * ep.swiglu_bound(C, D, bias, rel))
