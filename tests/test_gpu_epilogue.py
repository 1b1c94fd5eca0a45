"""GPU parity of the fused epilogue C := act(A.B + bias), run inside the
kernels' store phase, against the oracle's fp64 epilogue.

Acceptance per element (the oracle's fused-epilogue rule): |g - y| within
L * (1e-5 * D + 2^-22 |x|) + 2^-20 |y| (+ the smallest normal), with
x = C + bias, y = act(x), D = |A|.|B| and L the activation's Lipschitz
constant; a bf16 output must lie inside the RNE bracket of that interval.

Every compiled configuration of both kernels is forced in turn, so each
store path (staged tile epilogue, K-split store, skinny store) meets every
activation, with and without bias, fp32 and bf16 output, ragged edges and a
K tail. B is scaled so the products have unit variance and the activations
are exercised on both sides of their bends, not only where they saturate.
"""

import numpy as np
import pytest

import oracle
import tile_partitioned_dense_amd as tg
from tile_partitioned_dense_amd import synth

from gpu_helpers import Case, host_out, stream_tile_configs, tile_config_table, workload_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ACTS = [a for a in tg.Act if a != tg.Act.SWIGLU]     # elementwise activations
SKINNY_MG = [1, 1, 2, 2, 4, 4]


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    with tg.TileGemm(0) as gg:
        yield gg


def _bias(N, seed, scale=1.0):
    b = synth.draw_bias(N, seed, scale)
    return b, torch.from_numpy(b).to("cuda")


def _name(act):
    return tg.Act(act).name.lower()


def _combos():
    for act in ACTS:
        for with_bias in (True, False):
            if act == tg.Act.NONE and not with_bias:
                continue            # the plain product: covered by the parity tests
            yield act, with_bias


def _check_case(g, case, flags, bias_np, bias_dev, label):
    Cr, Dr = case.ref()
    for act, with_bias in _combos():
        for dt in (torch.float32, torch.bfloat16):
            store, C = case.out(dt)
            g.run_debug(case.A_dev, case.B_dev, C, flags=flags,
                        bias=bias_dev if with_bias else None, act=act)
            torch.cuda.synchronize()
            rep = oracle.check_epilogue(host_out(C), Cr, Dr, bias_np if with_bias else None,
                                        _name(act), out_bf16=dt == torch.bfloat16)
            assert rep.ok, f"{label} act={_name(act)} bias={with_bias} {dt}: {rep}"
            pad = store[:, case.N:]
            if pad.numel():
                assert torch.isnan(pad.float()).all(), f"{label}: store outside the owned columns"


def tile_shape(cfg):
    bm, bn = tile_config_table()[cfg][:2]
    return 2 * bm + 37, 2 * bn + 19


@pytest.mark.parametrize("cfg", range(tg.N_TILE_CONFIGS))
@pytest.mark.parametrize("bcol", [False, True], ids=["Brow", "Bcol"])
def test_tile_configs_epilogue(g, cfg, bcol):
    if cfg in stream_tile_configs() and not bcol:
        pytest.skip("stream configurations take a column-major B")
    M, N = tile_shape(cfg)
    K = 200
    print(f"[epilogue tile cfg {cfg} bcol={bcol} {M}x{N}x{K}]", flush=True)
    case = Case(M, N, K, bcol, seed=40 + cfg, pad=8, b_scale=K ** -0.5)
    b_np, b_dev = _bias(N, 700 + cfg)
    _check_case(g, case, tg.DEBUG_FORCE_TILE(cfg), b_np, b_dev, f"tile cfg {cfg}")


@pytest.mark.parametrize("cfg", range(tg.N_SKINNY_CONFIGS))
@pytest.mark.parametrize("bcol", [False, True], ids=["Brow", "Bcol"])
def test_skinny_configs_epilogue(g, cfg, bcol):
    M, N, K = 16 * SKINNY_MG[cfg] - 3, 16 * 8 * 5 + 13, 8 * 32 * 3 + 24 + 5
    print(f"[epilogue skinny cfg {cfg} bcol={bcol} {M}x{N}x{K}]", flush=True)
    case = Case(M, N, K, bcol, seed=60 + cfg, pad=8, b_scale=K ** -0.5)
    b_np, b_dev = _bias(N, 720 + cfg)
    _check_case(g, case, tg.DEBUG_FORCE_SKINNY(cfg), b_np, b_dev, f"skinny cfg {cfg}")


@pytest.mark.parametrize("M,N", [(300, 260), (5, 300)], ids=["tile", "skinny"])
def test_k_zero_gives_act_of_bias(g, M, N):
    """K = 0: the product is exactly zero, so every row is act(bias)."""
    print(f"[epilogue K=0 {M}x{N}]", flush=True)
    case = Case(M, N, 0, seed=80)
    b_np, b_dev = _bias(N, 740, scale=3.0)
    _check_case(g, case, 0, b_np, b_dev, "K=0")


@pytest.mark.parametrize("M,N,K", [(2048, 2304, 512), (4096, 256, 1024), (16, 4096, 2048)])
def test_bf16_epilogue_is_rne_of_fp32_epilogue(g, M, N, K):
    """One plan for both output types: the bf16 result is the RNE of the fp32
    result bit for bit, epilogue included (the conversion comes last)."""
    print(f"[epilogue rne {M}x{N}x{K}]", flush=True)
    case = Case(M, N, K, seed=90, b_scale=K ** -0.5)
    _, b_dev = _bias(N, 750)
    for act in (tg.Act.SILU, tg.Act.TANH):
        _, C32 = case.out(torch.float32)
        _, C16 = case.out(torch.bfloat16)
        g(case.A_dev, case.B_dev, C32, bias=b_dev, act=act)
        g(case.A_dev, case.B_dev, C16, bias=b_dev, act=act)
        torch.cuda.synchronize()
        f32 = host_out(C32).astype(np.float64)
        assert np.array_equal(host_out(C16), oracle.rne_bf16(f32)), _name(act)


def test_epilogue_is_deterministic(g):
    case = Case(1000, 1000, 1000, seed=91, b_scale=1000 ** -0.5)
    _, b_dev = _bias(1000, 751)
    outs = []
    for _ in range(5):
        _, C = case.out(torch.float32)
        g(case.A_dev, case.B_dev, C, bias=b_dev, act=tg.Act.SIGMOID)
        torch.cuda.synchronize()
        outs.append(C.view(torch.int32).clone())
    assert all(torch.equal(outs[0], o) for o in outs[1:])


def test_bad_epilogue_arguments_are_rejected(g):
    case = Case(64, 64, 64, seed=92)
    _, C = case.out(torch.float32)
    _, b = _bias(64, 752)
    st = tg.tile_gemm_run_epilogue(g.handle, case.A_dev, case.B_dev, C, bias=b, act=9,
                                   check=False)
    assert st == tg.Status.ERR_EPILOGUE
    st = tg.tile_gemm_run_epilogue(g.handle, case.A_dev, case.B_dev, C,
                                   bias=b.data_ptr() + 4, act=tg.Act.RELU, check=False)
    assert st == tg.Status.ERR_MISALIGNED
    assert torch.isnan(C).all(), "a rejected call launched nothing"


@pytest.mark.parametrize("name,act", [("mlp_gate_up_shard", tg.Act.SILU), ("decode", tg.Act.RELU),
                                      ("decode_colB", tg.Act.SIGMOID),
                                      ("qkv_shard", tg.Act.TANH)])
def test_workload_epilogue_sampled(g, name, act):
    """Full size, in the launch configuration the benchmark times: sampled
    elements against the oracle's one-element products plus its epilogue."""
    w, ops, A, B = workload_case(name)
    print(f"[epilogue workload {name} {w.M}x{w.N}x{w.K} act={_name(act)}]", flush=True)
    b_np, b_dev = _bias(w.N, 760)
    rng = np.random.default_rng(11)
    ii = np.concatenate([rng.integers(0, w.M, 300), [0, w.M - 1, 0, w.M - 1]])
    jj = np.concatenate([rng.integers(0, w.N, 300), [0, 0, w.N - 1, w.N - 1]])
    c, d = oracle.gemm_at(ops.A, ops.B, ii, jj)
    for dt in (torch.float32, torch.bfloat16):
        C = torch.full((w.M, w.N), float("nan"), dtype=dt, device="cuda")
        g(A, B, C, bias=b_dev, act=act)
        torch.cuda.synchronize()
        out = host_out(C)[ii, jj]
        rep = oracle.check_epilogue(out[None, :], c[None, :], d[None, :], b_np[jj],
                                    _name(act), out_bf16=dt == torch.bfloat16)
        assert rep.ok, f"{name} {dt}: {rep}"
        del C


# ------------------------------------------------------ SiLU(gate) * up

def _glu_out(case, dtype, pad=8):
    h = case.N // 2
    store = torch.full((case.M, h + pad), float("nan"), dtype=dtype, device="cuda")
    return store, store[:, :h]


def _check_glu(g, case, flags, bias_np, bias_dev, label, counts=False):
    Cr, Dr = case.ref()
    h = case.N // 2
    for with_bias in (True, False):
        for dt in (torch.float32, torch.bfloat16):
            store, C = _glu_out(case, dt)
            cnt = torch.zeros((case.M, h), dtype=torch.int32, device="cuda") if counts else None
            g.run_debug(case.A_dev, case.B_dev, C, counts=cnt,
                        flags=flags | (tg.DEBUG_COUNT_WRITES if counts else 0),
                        bias=bias_dev if with_bias else None, act=tg.Act.SWIGLU)
            torch.cuda.synchronize()
            rep = oracle.check_swiglu(host_out(C), Cr, Dr, bias_np if with_bias else None,
                                      out_bf16=dt == torch.bfloat16)
            assert rep.ok, f"{label} swiglu bias={with_bias} {dt}: {rep}"
            assert torch.isnan(store[:, h:].float()).all(), f"{label}: store outside C's columns"
            if counts:
                assert bool((cnt == 1).all()), f"{label}: an element not written exactly once"


@pytest.mark.parametrize("cfg", range(tg.N_TILE_CONFIGS))
@pytest.mark.parametrize("bcol", [False, True], ids=["Brow", "Bcol"])
def test_swiglu_tile_configs(g, cfg, bcol):
    if cfg in stream_tile_configs() and not bcol:
        pytest.skip("stream configurations take a column-major B")
    bm, bn = tile_config_table()[cfg][:2]
    M, N, K = 2 * bm + 37, 2 * (bn + 24), 200      # half = bn + 24: a ragged last tile
    print(f"[swiglu tile cfg {cfg} bcol={bcol} {M}x{N}x{K}]", flush=True)
    case = Case(M, N, K, bcol, seed=100 + cfg, pad=8, b_scale=K ** -0.5)
    b_np, b_dev = _bias(N, 800 + cfg)
    _check_glu(g, case, tg.DEBUG_FORCE_TILE(cfg), b_np, b_dev, f"tile cfg {cfg}", counts=True)


@pytest.mark.parametrize("cfg", range(tg.N_SKINNY_CONFIGS))
@pytest.mark.parametrize("bcol", [False, True], ids=["Brow", "Bcol"])
def test_swiglu_skinny_configs(g, cfg, bcol):
    M, N, K = 16 * SKINNY_MG[cfg] - 3, 2 * (8 * 8 * 3 + 8), 8 * 32 * 3 + 24 + 5
    print(f"[swiglu skinny cfg {cfg} bcol={bcol} {M}x{N}x{K}]", flush=True)
    case = Case(M, N, K, bcol, seed=120 + cfg, pad=8, b_scale=K ** -0.5)
    b_np, b_dev = _bias(N, 820 + cfg)
    _check_glu(g, case, tg.DEBUG_FORCE_SKINNY(cfg), b_np, b_dev, f"skinny cfg {cfg}",
               counts=True)


@pytest.mark.parametrize("M,N,K", [(300, 272, 0), (5, 304, 0), (1000, 1024, 1000),
                                   (64, 28672 // 8, 1024)], ids=["K0-tile", "K0-skinny",
                                                                  "square", "k-split"])
def test_swiglu_planner_path(g, M, N, K):
    print(f"[swiglu planner {M}x{N}x{K}]", flush=True)
    case = Case(M, N, K, seed=140, b_scale=max(K, 1) ** -0.5)
    b_np, b_dev = _bias(N, 840, scale=2.0)
    _check_glu(g, case, 0, b_np, b_dev, f"{M}x{N}x{K}")


def test_swiglu_rejects_bad_widths(g):
    case = Case(64, 72, 64, seed=141)                  # 72 is even but not a multiple of 16
    _, C = _glu_out(case, torch.float32)
    st = tg.tile_gemm_run_epilogue(g.handle, case.A_dev, case.B_dev, C, act=tg.Act.SWIGLU,
                                   check=False)
    assert st == tg.Status.ERR_BAD_SHAPE
    case = Case(64, 64, 64, seed=142)
    wrong = torch.empty((64, 64), dtype=torch.float32, device="cuda")   # must be 64 x 32
    with pytest.raises(ValueError):
        g(case.A_dev, case.B_dev, wrong, act=tg.Act.SWIGLU)


@pytest.mark.parametrize("name", ["mlp_gate_up_shard", "decode", "decode_colB"])
def test_swiglu_workload_sampled(g, name):
    """The gate+up workloads at full size with their SiLU(gate) * up: sampled
    output elements against the oracle's one-element products of both the
    gate and the up column."""
    w, ops, A, B = workload_case(name)
    h = w.N // 2
    print(f"[swiglu workload {name} {w.M}x{w.N}x{w.K}]", flush=True)
    b_np, b_dev = _bias(w.N, 860)
    rng = np.random.default_rng(12)
    ii = np.concatenate([rng.integers(0, w.M, 300), [0, w.M - 1, 0, w.M - 1]])
    jj = np.concatenate([rng.integers(0, h, 300), [0, 0, h - 1, h - 1]])
    cg, dg = oracle.gemm_at(ops.A, ops.B, ii, jj)
    cu, du = oracle.gemm_at(ops.A, ops.B, ii, jj + h)
    C2 = np.stack([cg, cu], axis=1)                     # n x 2: [gate, up] per sample
    D2 = np.stack([dg, du], axis=1)
    for dt in (torch.float32, torch.bfloat16):
        C = torch.full((w.M, h), float("nan"), dtype=dt, device="cuda")
        g(A, B, C, bias=b_dev, act=tg.Act.SWIGLU)
        torch.cuda.synchronize()
        out = host_out(C)[ii, jj]
        for t in range(len(ii)):
            bias2 = np.array([b_np[jj[t]], b_np[jj[t] + h]])
            rep = oracle.check_swiglu(out[t:t + 1, None], C2[t:t + 1], D2[t:t + 1], bias2,
                                      out_bf16=dt == torch.bfloat16)
            assert rep.ok, f"{name} {dt} sample ({ii[t]}, {jj[t]}): {rep}"
        del C
