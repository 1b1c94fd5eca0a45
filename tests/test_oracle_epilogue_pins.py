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
