"""GPU parity of the stream kernel (bf16, column-major B, few rows; the
planner's choice for column-major B, even K and M <= 64) against the fp64
oracle, through the C ABI.

The stream kernel moves K in stages of 128 or 256 values per row and zeroes, in
its last stage, every value at or past K; these cases put K on both sides of
stage and 8-value chunk boundaries, rows on both sides of the 32-row tile,
columns on both sides of the 128-column tile, and the owned tiles on one or
several workgroups. Acceptance as in test_gpu_parity: fp32 within
1e-5 * (|A|.|B|)_ij, bf16 inside the RNE bracket, integer inputs exact,
each element written once, nothing written outside C.
"""

import numpy as np
import pytest

import oracle
import tile_partitioned_dense_amd as tg
from tile_partitioned_dense_amd import synth

from gpu_helpers import Case, check, host_out, stream_tile_configs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

STREAM = sorted(stream_tile_configs())


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    with tg.TileGemm(0) as gg:
        yield gg


def _run_check(g, case, flags, integer=False, label=""):
    Cr, Dr = case.ref()
    for dt in (torch.float32, torch.bfloat16):
        store, C = case.out(dt)
        cnt = torch.zeros((case.M, case.N), dtype=torch.int32, device="cuda")
        g.run_debug(case.A_dev, case.B_dev, C, counts=cnt, flags=flags | tg.DEBUG_COUNT_WRITES)
        torch.cuda.synchronize()
        rep = check(host_out(C), Cr, Dr, dt == torch.bfloat16, integer)
        assert rep.ok, f"{label} {dt}: {rep}"
        assert bool((cnt == 1).all()), f"{label} {dt}: an element not written exactly once"
        if store.shape[1] > case.N:
            assert torch.isnan(store[:, case.N:].float()).all(), f"{label}: store outside C"


@pytest.mark.parametrize("cfg", STREAM)
@pytest.mark.parametrize("M,N,K", [
    (1, 1, 8),            # one value of K, one output
    (5, 300, 24),         # K inside the first chunk pair of one stage
    (16, 257, 128),       # exactly one stage
    (17, 383, 136),       # one stage and a chunk
    (32, 128, 1000),      # several stages, K % 16 == 8
    (40, 520, 1030),      # two tile rows, K % 8 == 6 (values masked inside a chunk)
    (9, 200, 2),          # the smallest even K
    (3, 1100, 2304),      # ring reused (18 stages)
    (64, 300, 520),       # the 64-row tile full
    (77, 260, 264),       # a second tile row of 64 rows
])
def test_stream_parity(g, cfg, M, N, K):
    print(f"[stream cfg {cfg} {M}x{N}x{K}]", flush=True)
    _run_check(g, Case(M, N, K, True, seed=M + N + K, pad=8), tg.DEBUG_FORCE_TILE(cfg),
               label=f"cfg {cfg} {M}x{N}x{K}")


@pytest.mark.parametrize("cfg", STREAM)
def test_stream_integer_exact(g, cfg):
    for M, N, K in ((7, 333, 518), (32, 260, 4098)):
        print(f"[stream int cfg {cfg} {M}x{N}x{K}]", flush=True)
        _run_check(g, Case(M, N, K, True, dist="int3", seed=K, pad=8), tg.DEBUG_FORCE_TILE(cfg),
                   integer=True, label=f"int cfg {cfg} {M}x{N}x{K}")


@pytest.mark.parametrize("cfg", STREAM)
def test_stream_several_tiles_per_workgroup_bit_identical(g, cfg):
    case = Case(70, 1300, 776, True, seed=91, pad=8)
    outs = []
    for flags in (0, tg.DEBUG_FORCE_GRID(3), tg.DEBUG_FORCE_GRID(7)):
        store, C = case.out(torch.float32)
        g.run_debug(case.A_dev, case.B_dev, C, flags=tg.DEBUG_FORCE_TILE(cfg) | flags)
        torch.cuda.synchronize()
        outs.append(C.clone())
    assert all(torch.equal(outs[0].view(torch.int32), o.view(torch.int32)) for o in outs[1:])
    Cr, Dr = case.ref()
    assert check(host_out(outs[0]), Cr, Dr, False).ok


def test_stream_deterministic_and_bf16_is_rne_of_fp32(g):
    case = Case(16, 4096, 4096, True, seed=92)
    outs = []
    for _ in range(5):
        _, C = case.out(torch.float32)
        g(case.A_dev, case.B_dev, C)
        torch.cuda.synchronize()
        outs.append(C.clone())
    assert all(torch.equal(outs[0].view(torch.int32), o.view(torch.int32)) for o in outs[1:])
    _, c16 = case.out(torch.bfloat16)
    g(case.A_dev, case.B_dev, c16)
    torch.cuda.synchronize()
    assert np.array_equal(host_out(c16), oracle.rne_bf16(host_out(outs[0]).astype(np.float64)))


@pytest.mark.parametrize("cfg", STREAM)
def test_stream_fused_epilogue(g, cfg):
    M, N, K = 21, 300, 520
    case = Case(M, N, K, True, seed=93, pad=8, b_scale=K ** -0.5)
    Cr, Dr = case.ref()
    b = synth.draw_bias(N, 94)
    bd = torch.from_numpy(b).cuda()
    for act in (tg.Act.NONE, tg.Act.RELU, tg.Act.SIGMOID, tg.Act.TANH, tg.Act.SILU):
        for dt in (torch.float32, torch.bfloat16):
            _, C = case.out(dt)
            g.run_debug(case.A_dev, case.B_dev, C, flags=tg.DEBUG_FORCE_TILE(cfg), bias=bd, act=act)
            torch.cuda.synchronize()
            rep = oracle.check_epilogue(host_out(C), Cr, Dr, b, act.name.lower(),
                                        out_bf16=dt == torch.bfloat16)
            assert rep.ok, f"{act.name} {dt}: {rep}"


@pytest.mark.parametrize("cfg", STREAM)
@pytest.mark.parametrize("M,N,K", [(16, 2 * 200, 264), (33, 2 * 128, 78)])
def test_stream_swiglu(g, cfg, M, N, K):
    """SiLU(gate) * up: the gate half of a tile and its up half come from
    B columns n0 .. and N/2 + n0 ..; ragged last tile (half = 200)."""
    case = Case(M, N, K, True, seed=95 + M, pad=8, b_scale=K ** -0.5)
    Cr, Dr = case.ref()
    b = synth.draw_bias(N, 96)
    bd = torch.from_numpy(b).cuda()
    h = N // 2
    for with_bias in (True, False):
        for dt in (torch.float32, torch.bfloat16):
            store = torch.full((M, h + 8), float("nan"), dtype=dt, device="cuda")
            C = store[:, :h]
            cnt = torch.zeros((M, h), dtype=torch.int32, device="cuda")
            g.run_debug(case.A_dev, case.B_dev, C, counts=cnt,
                        flags=tg.DEBUG_FORCE_TILE(cfg) | tg.DEBUG_COUNT_WRITES,
                        bias=bd if with_bias else None, act=tg.Act.SWIGLU)
            torch.cuda.synchronize()
            rep = oracle.check_swiglu(host_out(C), Cr, Dr, b if with_bias else None,
                                      out_bf16=dt == torch.bfloat16)
            assert rep.ok, f"swiglu bias={with_bias} {dt}: {rep}"
            assert bool((cnt == 1).all())
            assert torch.isnan(store[:, h:].float()).all()


@pytest.mark.parametrize("bcol,K", [(False, 256), (True, 255)], ids=["row-major B", "odd K"])
def test_stream_configuration_rejects_what_it_cannot_load(g, bcol, K):
    case = Case(16, 256, K, bcol, seed=97)
    _, C = case.out(torch.float32)
    st = tg.tile_gemm_run_debug(g.handle, case.A_dev, case.B_dev, C,
                                flags=tg.DEBUG_FORCE_TILE(STREAM[0]), check=False)
    assert st == tg.Status.ERR_BAD_SHAPE
    assert torch.isnan(C).all()


def test_odd_k_with_column_major_b_runs_elsewhere(g):
    """The planner keeps odd K off the stream kernel; the result is still
    right (the skinny kernel at 16 rows, the tile kernel's K-split
    configurations at 32)."""
    for M in (16, 32):
        p = tg.tile_gemm_plan(M, 700, 1031, True, 256)
        assert not (p.variant == tg.VARIANT_TILE and p.config in STREAM)
        _run_check(g, Case(M, 700, 1031, True, seed=98 + M, pad=8), 0, label=f"odd K {M} rows")
