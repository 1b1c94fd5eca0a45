"""The fused epilogue of the product, written for the oracle only.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed follows the epilogue fusion the TorchInductor page describes
("TorchInductor ganha suporte a GEMMs de alta performance com CuteDSL": the
paragraph on epilogue fusion, where a bias addition or an activation is folded
into the GEMM's store, and the roadmap paragraph listing element-wise
operations and the ReLU, sigmoid and tanh activations):

    out[i, j] = act(C[i, j] + bias[j])

with C the fp64 product, bias an optional length-N vector (absent: 0) and act
one of the plain definitions below, evaluated in fp64:

    none     x
    relu     max(x, 0)
    sigmoid  1 / (1 + e^-x)
    tanh     the hyperbolic tangent (numpy)
    silu     x * sigmoid(x)      (not on the pages; the usual definition)

Acceptance (check_epilogue): the GPU accumulates C in fp32 within tau =
rel * D (rel = 1e-5) of the exact product, adds the fp32 bias in fp32 and
evaluates act in fp32. With x = C + bias, the reference y = act(x) and L the
Lipschitz bound of act (none, relu, tanh: 1; sigmoid: 1/4; silu: 1.1), an fp32
result g must satisfy

    |g - y| <= L * (tau + 2^-22 |x|) + 2^-20 |y| + 2^-126,

the terms being the accumulation bound, the fp32 rounding of the bias add,
the fp32 evaluation of act (a few units in the last place) and an absolute
floor for results near zero. A bf16 result must lie within
[RNE(y - t), RNE(y + t)] for that same bound t (rounding is monotone).

SiLU(gate) * up (swiglu): the gated MLP step that follows the gate+up
projection of the LLM layers the pages shard (the merged gate+up weight of
the tensor-parallel page's column split). C is the M x N product of that
merged projection, N even, its first N/2 columns the gate and its last N/2
the up projection; with x = C + bias (bias of length N, optional)

    out[i, j] = silu(x[i, j]) * x[i, j + N/2],   0 <= j < N/2.

Acceptance (check_swiglu): with g, u the gate and up values of x, their
accumulation bounds tau_g, tau_u as above and e_g = tau_g + 2^-22 |g|,
e_u = tau_u + 2^-22 |u| (each operand's error before the activation),

    |out - y| <= 1.1 |u| e_g + |silu(g)| e_u + 1.1 e_g e_u + 2^-20 |y| + 2^-126,

first-order propagation through the product (silu's slope is at most 1.1)
plus the second-order term, the fp32 evaluation and the floor.
"""

from __future__ import annotations

import numpy as np

from .numerics import CheckReport, bf16_to_f64, rne_bf16, _first_bad

ACTS = ("none", "relu", "sigmoid", "tanh", "silu")
LIPSCHITZ = {"none": 1.0, "relu": 1.0, "sigmoid": 0.25, "tanh": 1.0, "silu": 1.1}


def act_f64(x, act: str) -> np.ndarray:
    """act(x) elementwise in fp64, by the definitions in the module docstring."""
    x = np.asarray(x, dtype=np.float64)
    if act == "none":
        return x.copy()
    if act == "relu":
        return np.maximum(x, 0.0)
    if act == "sigmoid":
        with np.errstate(over="ignore"):
            return 1.0 / (1.0 + np.exp(-x))
    if act == "tanh":
        return np.tanh(x)
    if act == "silu":
        with np.errstate(over="ignore"):
            return x / (1.0 + np.exp(-x))
    raise ValueError(f"unknown activation {act!r}")


def epilogue(C, bias=None, act: str = "none") -> np.ndarray:
    """act(C + bias) for an M x N fp64 product C and an optional length-N bias
    (float32 or float64 values, added to every row)."""
    C = np.asarray(C, dtype=np.float64)
    x = C if bias is None else C + np.asarray(bias, dtype=np.float64)[None, :]
    return act_f64(x, act)


def epilogue_bound(C, D, bias=None, act: str = "none", rel: float = 1e-5,
                   tau=None) -> np.ndarray:
    """The per-element tolerance t of the acceptance rule above. `tau`, when
    given, replaces rel * D as the product's own bound (a product computed
    with another arithmetic, such as the MX one, brings its own)."""
    C = np.asarray(C, dtype=np.float64)
    x = C if bias is None else C + np.asarray(bias, dtype=np.float64)[None, :]
    y = act_f64(x, act)
    tau = rel * np.asarray(D, dtype=np.float64) if tau is None else np.asarray(tau, dtype=np.float64)
    return LIPSCHITZ[act] * (tau + 2.0 ** -22 * np.abs(x)) + 2.0 ** -20 * np.abs(y) + 2.0 ** -126


def check_epilogue(g, C, D, bias=None, act: str = "none", out_bf16: bool = False,
                   rel: float = 1e-5, tau=None) -> CheckReport:
    """Check a GPU result g (fp32 values, or bf16 bit patterns when out_bf16)
    against act(C + bias) within epilogue_bound."""
    y = epilogue(C, bias, act)
    t = epilogue_bound(C, D, bias, act, rel, tau)
    if out_bf16:
        gb = np.asarray(g)
        lo = bf16_to_f64(rne_bf16(y - t))
        hi = bf16_to_f64(rne_bf16(y + t))
        gv = bf16_to_f64(gb)
        bad = ~((gv >= lo) & (gv <= hi))
        err = np.abs(gv - y)
    else:
        gv = np.asarray(g, dtype=np.float64)
        err = np.abs(gv - y)
        bad = ~(err <= t)
    ratio = float(np.max(err / t)) if err.size else 0.0
    return CheckReport(ok=not bool(bad.any()), n=int(bad.size), n_bad=int(bad.sum()),
                       max_ratio=ratio, first_bad=_first_bad(bad),
                       detail=f"act={act} bias={'yes' if bias is not None else 'no'}")


def swiglu(C, bias=None) -> np.ndarray:
    """silu(x[:, :N/2]) * x[:, N/2:] for x = C + bias (module docstring)."""
    C = np.asarray(C, dtype=np.float64)
    if C.shape[1] % 2:
        raise ValueError("swiglu needs an even number of product columns")
    x = C if bias is None else C + np.asarray(bias, dtype=np.float64)[None, :]
    h = C.shape[1] // 2
    return act_f64(x[:, :h], "silu") * x[:, h:]


def swiglu_bound(C, D, bias=None, rel: float = 1e-5) -> np.ndarray:
    """The per-element tolerance of check_swiglu (module docstring)."""
    C = np.asarray(C, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    x = C if bias is None else C + np.asarray(bias, dtype=np.float64)[None, :]
    h = C.shape[1] // 2
    g, u = x[:, :h], x[:, h:]
    eg = rel * D[:, :h] + 2.0 ** -22 * np.abs(g)
    eu = rel * D[:, h:] + 2.0 ** -22 * np.abs(u)
    sg = act_f64(g, "silu")
    y = sg * u
    return (1.1 * np.abs(u) * eg + np.abs(sg) * eu + 1.1 * eg * eu + 2.0 ** -20 * np.abs(y)
            + 2.0 ** -126)


def check_swiglu(g, C, D, bias=None, out_bf16: bool = False, rel: float = 1e-5) -> CheckReport:
    """Check a GPU swiglu result g (M x N/2; fp32 values, or bf16 bit patterns
    when out_bf16) against swiglu(C, bias) within swiglu_bound."""
    y = swiglu(C, bias)
    t = swiglu_bound(C, D, bias, rel)
    if out_bf16:
        gv = bf16_to_f64(np.asarray(g))
        lo = bf16_to_f64(rne_bf16(y - t))
        hi = bf16_to_f64(rne_bf16(y + t))
        bad = ~((gv >= lo) & (gv <= hi))
    else:
        gv = np.asarray(g, dtype=np.float64)
        bad = ~(np.abs(gv - y) <= t)
    err = np.abs(gv - y)
    ratio = float(np.max(err / t)) if err.size else 0.0
    return CheckReport(ok=not bool(bad.any()), n=int(bad.size), n_bad=int(bad.sum()),
                       max_ratio=ratio, first_bad=_first_bad(bad),
                       detail=f"swiglu bias={'yes' if bias is not None else 'no'}")
