"""GPU parity of the MXFP8 product (tile_gemm_run_mx) against the oracle's
microscaled product (oracle/mx.py), through the C ABI.

Acceptance, first and device-independent: integer-valued elements, with unit
scales or with every block's E8M0 scale drawn from a range (the product
exponents then span 6, so every partial sum is exact in fp32 in any order and
the result is the exact sum), must equal the oracle exactly, on every
configuration, both formats and the full-size workloads. Then, for random
operands: fp32 output within the oracle's per-element MX bound T of the fp64
sum (a model of the instruction's grouped fixed-point summation, see
oracle/mx.py), bf16 output inside the RNE bracket of that interval. Outputs
start as NaN (padding columns included) and a write counter checks that
every element is written exactly once.
"""

import numpy as np
import pytest

import oracle
import tile_partitioned_dense_amd as tg
from tile_partitioned_dense_amd import synth

from gpu_helpers import host_out

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    with tg.TileGemm(0) as gg:
        yield gg


def _mx_config_rows():
    import os
    import re
    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "tile_partitioned_dense_amd", "csrc", "plan.hpp")).read()
    body = re.search(r"kMxConfigs\[kNumMxConfigs\]\s*=\s*\{(.*?)\n\};", src, re.S).group(1)
    return [[f.strip() for f in r.split(",")] for r in re.findall(r"^\s*\{([^}]*)\}", body, re.M)]


def mx_config_table():
    """(bm, bn) of every MX configuration, in index order."""
    return [(int(r[0]), int(r[1])) for r in _mx_config_rows()]


def mx_stream_configs():
    """(index, bm, bn, stages, bytes of K per row and stage) of the stream-kernel
    configurations."""
    return [(i, int(r[0]), int(r[1]), int(r[4]), int(r[6])) for i, r in enumerate(_mx_config_rows())
            if len(r) > 6 and int(r[6]) > 0]


def mx_k_unit(cfg, fmt):
    """K values per slab of a configuration: 128 for E2M1 and for the
    16x16x128 configurations (their K steps), else 64."""
    r = _mx_config_rows()[cfg]
    return 128 if fmt == "e2m1" or (len(r) > 9 and int(r[9]) == 16) else 64


FMTS = {"e4m3": tg.MX_E4M3, "e2m1": tg.MX_E2M1}


class MxCase:
    def __init__(self, M, N, K, dist="normal", seed=0, pad=16, b_scale=1.0, fmt="e4m3",
                 varied_scales=False):
        self.M, self.N, self.K, self.fmt = M, N, K, fmt
        fp4 = fmt == "e2m1"
        kb = K // 2 if fp4 else K                      # bytes of K in a row
        lk = K + (2 * pad if fp4 else pad)             # padded rows (16 more bytes)
        sca = synth.MX_INT_SCALES_A if varied_scales else None
        scb = synth.MX_INT_SCALES_B if varied_scales else None
        A, sA = synth.draw_mx(M, lk, dist, 2 * seed + 1, fmt=fmt, scale_codes=sca)
        Bt, sB = synth.draw_mx(N, lk, dist, 2 * seed + 2, b_scale, fmt=fmt, scale_codes=scb)
        ls = synth.mx_scale_stride(K)
        self.A, self.Bt = A[:, :kb], Bt[:, :kb]
        K = kb
        self.sA, self.sB = sA[:, :ls], sB[:, :ls]
        dA = torch.from_numpy(A).cuda()
        dB = torch.from_numpy(Bt).cuda()
        self.A_dev, self.Bt_dev = dA[:, :K], dB[:, :K]
        self.sA_dev = torch.from_numpy(np.ascontiguousarray(self.sA)).cuda()
        self.sB_dev = torch.from_numpy(np.ascontiguousarray(self.sB)).cuda()
        self._ref = None

    def ref(self):
        if self._ref is None:
            self._ref = oracle.mx.mx_gemm(self.A, self.sA, self.Bt, self.sB, self.K, self.fmt)
        return self._ref

    def bound(self):
        if getattr(self, "_bound", None) is None:
            self._bound = oracle.mx.mx_bound(self.A, self.sA, self.Bt, self.sB, self.K, self.fmt)
        return self._bound

    def out(self, dtype, pad=8):
        ld = (self.N + 7) // 8 * 8 + pad                # 16-byte rows for both output types
        store = torch.full((self.M, ld), float("nan"), dtype=dtype, device="cuda")
        return store, store[:, : self.N]


def _check(out, C, T, bf16, integer=False):
    if integer:
        return oracle.check_exact(out, C, bf16)
    return oracle.mx.check_mx(out, C, T, out_bf16=bf16)


def _run_and_check(g, case, flags=0, integer=False, label=""):
    C, _ = case.ref()
    D = case.bound()
    for dt in (torch.float32, torch.bfloat16):
        store, out = case.out(dt)
        cnt = torch.zeros((case.M, case.N), dtype=torch.int32, device="cuda")
        g.mx(case.A_dev, case.Bt_dev, out, case.sA_dev, case.sB_dev, counts=cnt,
             flags=flags | tg.DEBUG_COUNT_WRITES, fmt=FMTS[case.fmt])
        torch.cuda.synchronize()
        rep = _check(host_out(out), C, D, dt == torch.bfloat16, integer)
        assert rep.ok, f"{label} {dt}: {rep}"
        assert bool((cnt == 1).all()), f"{label} {dt}: an element not written exactly once"
        assert torch.isnan(store[:, case.N:].float()).all(), f"{label}: store outside C"


@pytest.mark.parametrize("fmt", sorted(FMTS))
@pytest.mark.parametrize("cfg", range(tg.N_MX_CONFIGS))
@pytest.mark.parametrize("slabs", [1, 3, 4, 19])
def test_mx_configs(g, fmt, cfg, slabs):
    """Every configuration and format; 19 slabs run the steady loop and reuse
    the LDS scale windows."""
    bm, bn = mx_config_table()[cfg]
    M, N = 2 * bm + 37, 2 * bn + 19
    K = slabs * mx_k_unit(cfg, fmt)
    print(f"[mx {fmt} cfg {cfg} {M}x{N}x{K}]", flush=True)
    _run_and_check(g, MxCase(M, N, K, seed=cfg * 10 + slabs, fmt=fmt), tg.DEBUG_FORCE_TILE(cfg),
                   label=f"{fmt} cfg {cfg}")


@pytest.mark.parametrize("fmt", sorted(FMTS))
@pytest.mark.parametrize("cfg", range(tg.N_MX_CONFIGS))
def test_mx_configs_integer_exact(g, fmt, cfg):
    bm, bn = mx_config_table()[cfg]
    M, N, K = bm + 5, bn + 3, 640
    print(f"[mx int {fmt} cfg {cfg} {M}x{N}x{K}]", flush=True)
    _run_and_check(g, MxCase(M, N, K, dist="int3", seed=50 + cfg, fmt=fmt),
                   tg.DEBUG_FORCE_TILE(cfg), integer=True, label=f"int {fmt} cfg {cfg}")


@pytest.mark.parametrize("fmt", sorted(FMTS))
@pytest.mark.parametrize("cfg", range(tg.N_MX_CONFIGS))
def test_mx_configs_scaled_integer_exact(g, fmt, cfg):
    """Integer elements with per-block scales that vary along K and across
    rows (A's bytes 120..123, B's 131..134): exact, so every scale is applied
    to exactly its own block, whatever the arithmetic inside the instruction.
    19 slabs run the steady loop and reuse the LDS scale windows; two tile rows
    and columns plus ragged edges."""
    bm, bn = mx_config_table()[cfg]
    M, N = 2 * bm + 37, 2 * bn + 19
    K = 19 * mx_k_unit(cfg, fmt)
    print(f"[mx scaled int {fmt} cfg {cfg} {M}x{N}x{K}]", flush=True)
    case = MxCase(M, N, K, dist="int3", seed=80 + cfg, fmt=fmt, varied_scales=True)
    _run_and_check(g, case, tg.DEBUG_FORCE_TILE(cfg), integer=True,
                   label=f"scaled int {fmt} cfg {cfg}")


@pytest.mark.parametrize("fmt", sorted(FMTS))
@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (16, 4096, 1024), (64, 1000, 2048),
                                   (1000, 1000, 1024)])
def test_mx_planner_scaled_integer_exact(g, fmt, M, N, K):
    print(f"[mx planner scaled int {fmt} {M}x{N}x{K}]", flush=True)
    case = MxCase(M, N, K, dist="int3", seed=M + N, fmt=fmt, varied_scales=True)
    _run_and_check(g, case, integer=True, label=f"planner scaled int {fmt} {M}x{N}x{K}")


@pytest.mark.parametrize("name", sorted(synth.MX_WORKLOADS))
def test_mx_workload_scaled_integer_exact(g, name):
    """Full size, in the launch configuration the benchmark times, every
    element: integer codes with varied per-block scales, exact."""
    w = synth.MX_WORKLOADS[name]
    ops = synth.mx_operands(w, integer=True, varied_scales=True)
    print(f"[mx workload scaled int {name} {w.M}x{w.N}x{w.K}]", flush=True)
    A, Bt = torch.from_numpy(ops.A).cuda(), torch.from_numpy(ops.Bt).cuda()
    sA, sB = torch.from_numpy(ops.sA).cuda(), torch.from_numpy(ops.sB).cuda()
    C64, _ = oracle.mx.mx_gemm(ops.A, ops.sA, ops.Bt, ops.sB, w.K, w.fmt, want_d=False)
    for dt in (torch.float32, torch.bfloat16):
        C = torch.full((w.M, w.N), float("nan"), dtype=dt, device="cuda")
        g.mx(A, Bt, C, sA, sB, fmt=FMTS[w.fmt])
        torch.cuda.synchronize()
        rep = oracle.check_exact(host_out(C), C64, dt == torch.bfloat16)
        assert rep.ok, f"{name} {dt}: {rep}"
        del C


@pytest.mark.parametrize("fmt", sorted(FMTS))
@pytest.mark.parametrize("cfg,bm,bn,stages,sb", mx_stream_configs())
def test_mx_stream_ring(g, fmt, cfg, bm, bn, stages, sb):
    """Stream kernel over many stages: the stage ring and the scale-window
    ring are each reused several times, the last stage is only partly inside
    K, two tile rows (M > bm) and a ragged last tile column."""
    slabs = (sb // 64) * (stages + 3) + 3
    M, N = bm + 3, 3 * bn + 5
    K = slabs * (128 if fmt == "e2m1" else 64)
    print(f"[mx stream {fmt} cfg {cfg} {M}x{N}x{K}]", flush=True)
    _run_and_check(g, MxCase(M, N, K, seed=70 + cfg, fmt=fmt), tg.DEBUG_FORCE_TILE(cfg),
                   label=f"stream {fmt} cfg {cfg}")


@pytest.mark.parametrize("fmt", sorted(FMTS))
@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (17, 33, 128), (300, 520, 640), (16, 4096, 1024),
                                   (1000, 1000, 1024), (130, 130, 0)])
def test_mx_planner_shapes(g, fmt, M, N, K):
    print(f"[mx planner {fmt} {M}x{N}x{K}]", flush=True)
    case = MxCase(M, N, K, seed=M + N + K, fmt=fmt)
    _run_and_check(g, case, label=f"{fmt} {M}x{N}x{K}")


def test_mx_several_tiles_per_workgroup(g):
    case = MxCase(600, 700, 256, seed=61)
    print("[mx forced grid]", flush=True)
    for cfg, grid in ((0, 3), (1, 5), (3, 3), (4, 2)):
        _run_and_check(g, case, tg.DEBUG_FORCE_TILE(cfg) | tg.DEBUG_FORCE_GRID(grid),
                       label=f"cfg {cfg} grid {grid}")


@pytest.mark.parametrize("M", [300, 16])
def test_mx_fused_epilogue(g, M):
    """Tile kernel (300 rows) and stream kernel (16 rows, the planner's choice)."""
    case = MxCase(M, 264, 512, seed=62, b_scale=512 ** -0.5)
    C, D = case.ref()
    b = synth.draw_bias(case.N, 900)
    bd = torch.from_numpy(b).cuda()
    for act in (tg.Act.RELU, tg.Act.SILU, tg.Act.TANH):
        for dt in (torch.float32, torch.bfloat16):
            _, out = case.out(dt)
            g.mx(case.A_dev, case.Bt_dev, out, case.sA_dev, case.sB_dev, bias=bd, act=act)
            torch.cuda.synchronize()
            rep = oracle.check_epilogue(host_out(out), C, D, b, act.name.lower(),
                                        out_bf16=dt == torch.bfloat16, tau=case.bound())
            assert rep.ok, f"{act.name} {dt}: {rep}"


@pytest.mark.parametrize("fmt", sorted(FMTS))
@pytest.mark.parametrize("cfg", [i for i, r in enumerate(_mx_config_rows()) if not (len(r) > 6 and int(r[6]) > 0)])
def test_mx_fused_epilogue_every_tile_config(g, fmt, cfg):
    """bias + activation in the store of every MX tile configuration (forced),
    ragged in both dimensions, against the oracle's epilogue."""
    bm, bn = mx_config_table()[cfg]
    case = MxCase(bm + 37, bn + 19, 4 * mx_k_unit(cfg, fmt), seed=70 + cfg, fmt=fmt,
                  b_scale=512 ** -0.5)
    print(f"[mx epilogue {fmt} cfg {cfg} {case.M}x{case.N}x{case.K}]", flush=True)
    C, D = case.ref()
    b = synth.draw_bias(case.N, 901)
    bd = torch.from_numpy(b).cuda()
    for act in (tg.Act.RELU, tg.Act.SILU):
        for dt in (torch.float32, torch.bfloat16):
            _, out = case.out(dt)
            g.mx(case.A_dev, case.Bt_dev, out, case.sA_dev, case.sB_dev, bias=bd, act=act,
                 flags=tg.DEBUG_FORCE_TILE(cfg), fmt=FMTS[fmt])
            torch.cuda.synchronize()
            rep = oracle.check_epilogue(host_out(out), C, D, b, act.name.lower(),
                                        out_bf16=dt == torch.bfloat16, tau=case.bound())
            assert rep.ok, f"cfg {cfg} {fmt} {act.name} {dt}: {rep}"


def test_mx_deterministic_and_bf16_is_rne_of_fp32(g):
    case = MxCase(1024, 1024, 2048, seed=63)
    outs = []
    for _ in range(5):
        _, out = case.out(torch.float32)
        g.mx(case.A_dev, case.Bt_dev, out, case.sA_dev, case.sB_dev)
        torch.cuda.synchronize()
        outs.append(out.clone())
    assert all(torch.equal(outs[0].view(torch.int32), o.view(torch.int32)) for o in outs[1:])
    _, o16 = case.out(torch.bfloat16)
    g.mx(case.A_dev, case.Bt_dev, o16, case.sA_dev, case.sB_dev)
    torch.cuda.synchronize()
    assert np.array_equal(host_out(o16), oracle.rne_bf16(host_out(outs[0]).astype(np.float64)))


def test_mx_rejects_bad_arguments(g):
    case = MxCase(64, 64, 128, seed=64)
    _, out = case.out(torch.float32)
    A96 = case.A_dev[:, :96]
    B96 = case.Bt_dev[:, :96]
    st = tg.tile_gemm_run_mx(g.handle, A96, B96, out, case.sA_dev, case.sB_dev, check=False)
    assert st == tg.Status.ERR_BAD_SHAPE                 # K not a multiple of 64
    st = tg.tile_gemm_run_mx(g.handle, case.A_dev, case.Bt_dev, out, case.sA_dev, case.sB_dev,
                             act=tg.Act.SWIGLU, check=False)
    assert st == tg.Status.ERR_EPILOGUE
    assert torch.isnan(out).all()


@pytest.mark.parametrize("name", sorted(synth.MX_WORKLOADS))
def test_mx_workload_sampled(g, name):
    fmt = synth.MX_WORKLOADS[name].fmt
    """Full size, in the launch configuration the benchmark times: sampled
    elements against the oracle's one-element sums."""
    w = synth.MX_WORKLOADS[name]
    ops = synth.mx_operands(w)
    print(f"[mx workload {name} {w.M}x{w.N}x{w.K}]", flush=True)
    A, Bt = torch.from_numpy(ops.A).cuda(), torch.from_numpy(ops.Bt).cuda()
    sA, sB = torch.from_numpy(ops.sA).cuda(), torch.from_numpy(ops.sB).cuda()
    rng = np.random.default_rng(13)
    ii = np.concatenate([rng.integers(0, w.M, 200), [0, w.M - 1, 0, w.M - 1]])
    jj = np.concatenate([rng.integers(0, w.N, 200), [0, 0, w.N - 1, w.N - 1]])
    c, d = oracle.mx.mx_gemm_at(ops.A, ops.sA, ops.Bt, ops.sB, w.K, ii, jj, fmt)
    t = oracle.mx.mx_bound_at(ops.A, ops.sA, ops.Bt, ops.sB, w.K, ii, jj, fmt)
    for dt in (torch.float32, torch.bfloat16):
        C = torch.full((w.M, w.N), float("nan"), dtype=dt, device="cuda")
        g.mx(A, Bt, C, sA, sB, fmt=FMTS[fmt])
        torch.cuda.synchronize()
        out = host_out(C)
        assert not np.isnan(out.astype(np.float32) if dt == torch.float32 else
                            oracle.bf16_to_f64(out)).any(), "an element was not written"
        rep = oracle.mx.check_mx(out[ii, jj], c, t, out_bf16=dt == torch.bfloat16)
        assert rep.ok, f"{name} {dt}: {rep}"
        del C


def test_mx_16x16_configuration_rejects_k_not_a_multiple_of_128(g):
    """The 16x16x128 configurations take K in steps of 128; forced onto an
    E4M3 product whose K is only a multiple of 64 they refuse it (the
    planner never picks them for such a K)."""
    cfg = next(i for i, r in enumerate(_mx_config_rows()) if len(r) > 9 and int(r[9]) == 16)
    case = MxCase(300, 260, 192, seed=7)
    _, out = case.out(torch.float32)
    with pytest.raises(tg.TileGemmError) as e:
        g.mx(case.A_dev, case.Bt_dev, out, case.sA_dev, case.sB_dev, flags=tg.DEBUG_FORCE_TILE(cfg))
    assert "multiple of 128" in str(e.value)
    p = tg.tile_gemm_plan_mx(300, 7168, 192, tg.MX_E4M3)
    assert p.config != cfg
