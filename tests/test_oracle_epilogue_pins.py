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
