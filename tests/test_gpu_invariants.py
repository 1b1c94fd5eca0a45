"""GPU invariants of the partition discipline:

* bit-identical results over 10 runs (the pages report 17-35% of elements
  differing run to run when two tile programs share a destination; here the
  fraction must be 0) -- "GPU speed, without leaving Rust's safety model",
  section "Disjointness outside. Ordering inside.";
* every element written exactly once (a test-only write counter) and no NaN
  sentinel left behind;
* a deliberately colliding tile map (negative control) is caught by the same
  checks;
* argument errors return before launch and leave C untouched;
* work goes to the caller's stream.
"""

import ctypes

import numpy as np
import pytest

import tile_partitioned_dense_amd as tg
from tile_partitioned_dense_amd import synth

from gpu_helpers import Case, check, host_out, stream_tile_configs, workload_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    with tg.TileGemm(0) as gg:
        yield gg


def _as_int(C):
    return C.view(torch.int32) if C.dtype == torch.float32 else C.view(torch.int16)


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_ten_runs_bit_identical(g, name):
    w, ops, A, B = workload_case(name)
    dt = torch.bfloat16 if "bf16" in w.outs and "f32" not in w.outs else torch.float32
    print(f"[determinism {name} {dt}]", flush=True)
    ref = torch.empty((w.M, w.N), dtype=dt, device="cuda")
    g(A, B, ref)
    scratch = torch.empty_like(ref)
    differing = 0
    for _ in range(10):
        scratch.fill_(float("nan"))
        g(A, B, scratch)
        differing += int((_as_int(scratch) != _as_int(ref)).sum().item())
    torch.cuda.synchronize()
    frac = differing / (10 * ref.numel())
    print(f"  fraction of elements differing across 10 runs: {frac}", flush=True)
    assert differing == 0


def _counts_run(g, case, dt, flags):
    store, C = case.out(dt)
    counts = torch.zeros((case.M, case.N), dtype=torch.int32, device="cuda")
    g.run_debug(case.A_dev, case.B_dev, C, counts=counts, flags=flags)
    torch.cuda.synchronize()
    return store, C, counts


@pytest.mark.parametrize("M,N,K,bcol", [
    (1000, 1000, 200, False), (1000, 1000, 200, True), (40, 3000, 500, False),
    (40, 3000, 500, True), (16, 28672, 256, False), (8192, 1280, 64, False),
    (8192, 7168, 64, True), (4096, 4096, 64, False), (256, 256, 256, False)])
def test_every_element_written_once(g, M, N, K, bcol):
    print(f"[write-once {M}x{N}x{K} bcol={bcol}]", flush=True)
    case = Case(M, N, K, bcol, seed=7, pad=8)
    for dt in (torch.float32, torch.bfloat16):
        store, C, counts = _counts_run(g, case, dt, tg.DEBUG_COUNT_WRITES)
        assert int(counts.min()) == 1 and int(counts.max()) == 1
        assert not torch.isnan(C.float()).any()
        assert torch.isnan(store[:, N:].float()).all()


@pytest.mark.parametrize("cfg", range(tg.N_TILE_CONFIGS))
def test_every_config_writes_once(g, cfg):
    case = Case(300, 500, 70, cfg in stream_tile_configs(), seed=cfg)
    store, C, counts = _counts_run(g, case, torch.float32,
                                   tg.DEBUG_COUNT_WRITES | tg.DEBUG_FORCE_TILE(cfg))
    assert int(counts.min()) == 1 and int(counts.max()) == 1


@pytest.mark.parametrize("cfg,grid", [(1, 1), (1, 3), (7, 2), (9, 5), (6, 8), (10, 3), (11, 5), (12, 3),
                                      (14, 3), (14, 7), (15, 5)])
def test_workgroups_owning_several_tiles(g, cfg, grid):
    """A launch with fewer workgroups than tiles (workgroup w owns tile
    numbers w, w + grid, ...): every element still written once, and the
    result bit-identical to one workgroup per tile, since each tile keeps its
    own K loop and K order whichever workgroup runs it."""
    case = Case(700, 900, 300, cfg in (1, 9) or cfg in stream_tile_configs(), seed=40 + cfg,
                pad=8)                                             # steady loop + K tail
    print(f"[several tiles per workgroup cfg {cfg} grid {grid}]", flush=True)
    for dt in (torch.float32, torch.bfloat16):
        store, C, counts = _counts_run(g, case, dt, tg.DEBUG_COUNT_WRITES | tg.DEBUG_FORCE_TILE(cfg)
                                       | tg.DEBUG_FORCE_GRID(grid))
        assert int(counts.min()) == 1 and int(counts.max()) == 1
        assert not torch.isnan(C.float()).any()
        assert torch.isnan(store[:, case.N:].float()).all()
        _, C1, _ = _counts_run(g, case, dt, tg.DEBUG_FORCE_TILE(cfg) | tg.DEBUG_ONE_TILE_PER_WG)
        assert torch.equal(_as_int(C), _as_int(C1))
        Cr, Dr = case.ref()
        rep = check(host_out(C), Cr, Dr, dt == torch.bfloat16, False)
        assert rep.ok, rep


@pytest.mark.parametrize("cfg", [26, 27, 28])
@pytest.mark.parametrize("K", [512, 500])
@pytest.mark.parametrize("bcol", [True, False])
def test_one_wave_per_simd_tiles_several_per_workgroup(g, cfg, K, bcol):
    """The one-wave-per-SIMD 64-deep configurations with several tiles per
    workgroup (eight slabs, the last one through the register path when
    K = 500): every element written once, exactly the one-tile-per-workgroup
    result and the oracle's, for the plain store and for a fused bias + SiLU
    (the steady loop, the slab-at-a-time tail and the store all run again for
    each of a workgroup's tiles)."""
    case = Case(700, 900, K, bcol, seed=60 + cfg, pad=8)
    print(f"[several tiles one wave per SIMD cfg {cfg} K {K} bcol {bcol}]", flush=True)
    Cr, Dr = case.ref()
    for dt in (torch.float32, torch.bfloat16):
        store, C, counts = _counts_run(g, case, dt, tg.DEBUG_COUNT_WRITES | tg.DEBUG_FORCE_TILE(cfg)
                                       | tg.DEBUG_FORCE_GRID(3))
        assert int(counts.min()) == 1 and int(counts.max()) == 1
        assert torch.isnan(store[:, case.N:].float()).all()
        _, C1, _ = _counts_run(g, case, dt, tg.DEBUG_FORCE_TILE(cfg) | tg.DEBUG_ONE_TILE_PER_WG)
        assert torch.equal(_as_int(C), _as_int(C1))
        rep = check(host_out(C), Cr, Dr, dt == torch.bfloat16, False)
        assert rep.ok, rep
        bias = torch.linspace(-1.0, 1.0, case.N, dtype=torch.float32, device="cuda")
        outs = []
        for fl in (tg.DEBUG_FORCE_GRID(3), tg.DEBUG_ONE_TILE_PER_WG):
            _, Ce = case.out(dt)
            g.run_debug(case.A_dev, case.B_dev, Ce, flags=tg.DEBUG_FORCE_TILE(cfg) | fl, bias=bias,
                        act=tg.Act.SILU)
            torch.cuda.synchronize()
            outs.append(Ce)
        assert torch.equal(_as_int(outs[0]), _as_int(outs[1]))


def test_forced_grid_rejected_for_the_skinny_kernel(g):
    case = Case(16, 512, 64, False, seed=3)
    store, C = case.out(torch.float32)
    with pytest.raises(tg.TileGemmError):
        g.run_debug(case.A_dev, case.B_dev, C, flags=tg.DEBUG_FORCE_GRID(2))
    torch.cuda.synchronize()
    assert torch.isnan(C).all()


@pytest.mark.parametrize("cfg", range(tg.N_SKINNY_CONFIGS))
def test_every_skinny_config_writes_once(g, cfg):
    case = Case(13, 1500, 333, False, seed=cfg)
    store, C, counts = _counts_run(g, case, torch.float32,
                                   tg.DEBUG_COUNT_WRITES | tg.DEBUG_FORCE_SKINNY(cfg))
    assert int(counts.min()) == 1 and int(counts.max()) == 1


def test_negative_control_collision_is_caught(g):
    """Workgroup 1 is made to take workgroup 0's tile: one tile is written
    twice and another never. The write counter and the sentinel both see it."""
    case = Case(1024, 1024, 128, False, seed=3)
    store, C, counts = _counts_run(g, case, torch.float32,
                                   tg.DEBUG_COUNT_WRITES | tg.DEBUG_COLLIDE)
    cnt = counts.cpu().numpy()
    assert cnt.max() == 2 and cnt.min() == 0
    plan = tg.tile_gemm_plan(1024, 1024, 128, False, 256)
    assert (cnt == 2).sum() == plan.bm * plan.bn == (cnt == 0).sum()
    assert torch.isnan(C).sum().item() == plan.bm * plan.bn


def test_errors_leave_output_untouched(g):
    case = Case(128, 128, 64, False, seed=5)
    store, C = case.out(torch.float32, fill=7.0)
    s = tg.Strides(case.A_dev.stride(0), 1, case.B_dev.stride(0), 1, C.stride(0), 1)
    h = g.handle
    # misaligned A pointer
    st = tg.tile_gemm_run(h, case.A_dev.data_ptr() + 2, case.B_dev.data_ptr(), C.data_ptr(),
                          128, 128, 64, s, tg.Dtype.BF16_TO_F32, None, check=False)
    assert st == tg.Status.ERR_MISALIGNED
    # C aliasing A
    st = tg.tile_gemm_run(h, case.A_dev.data_ptr(), case.B_dev.data_ptr(),
                          case.A_dev.data_ptr(), 128, 128, 64, s, tg.Dtype.BF16_TO_F32, None,
                          check=False)
    assert st == tg.Status.ERR_ALIAS
    # unknown dtype
    st = tg.tile_gemm_run(h, case.A_dev.data_ptr(), case.B_dev.data_ptr(), C.data_ptr(),
                          128, 128, 64, s, 5, None, check=False)
    assert st == tg.Status.ERR_DTYPE
    torch.cuda.synchronize()
    assert bool((store == 7.0).all())


def test_runs_on_the_callers_stream(g):
    case = Case(512, 512, 256, False, seed=6)
    Cr, _ = case.ref()
    side = torch.cuda.Stream()
    store, C = case.out(torch.float32)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        g(case.A_dev, case.B_dev, C)           # binding picks up the current stream
    side.synchronize()
    out = host_out(C)
    assert np.all(np.abs(out - Cr) <= 1e-5 * case.ref()[1])


def test_handle_checks_current_device(g):
    lib = tg.load_library()
    h = ctypes.c_void_p()
    assert lib.tile_gemm_create(ctypes.byref(h), 10_000) == tg.Status.ERR_DEVICE
    assert lib.tile_gemm_create(ctypes.byref(h), 0) == tg.Status.OK
    assert lib.tile_gemm_destroy(h) == tg.Status.OK


def test_plan_log_prints_each_shape_once(capfd, monkeypatch):
    """TILE_GEMM_LOG=1 (read at create) prints the launched plan to stderr once
    per call shape, and the printed plan is the planner's."""
    monkeypatch.setenv("TILE_GEMM_LOG", "1")
    with tg.TileGemm(0) as lg:
        cases = [(300, 264, 200), (16, 512, 256)]
        for M, N, K in cases + cases[:1]:
            A = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
            B = torch.zeros((K, N), dtype=torch.bfloat16, device="cuda")
            C = torch.empty((M, N), dtype=torch.float32, device="cuda")
            lg(A, B, C)
        torch.cuda.synchronize()
    err = capfd.readouterr().err
    lines = [ln for ln in err.splitlines() if ln.startswith("tile_gemm: run ")]
    assert len(lines) == 2, err
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    for (M, N, K), ln in zip(cases, lines):
        p = tg.tile_gemm_plan(M, N, K, False, cu)
        assert f" M={M} N={N} K={K} B=row-major" in ln, ln
        assert f" config {p.config}, tile {p.bm}x{p.bn}," in ln and f" grid {p.grid}," in ln, ln


def test_plan_log_off_by_default(capfd, monkeypatch):
    monkeypatch.delenv("TILE_GEMM_LOG", raising=False)
    with tg.TileGemm(0) as lg:
        A = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
        B = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
        C = torch.empty((64, 64), dtype=torch.float32, device="cuda")
        lg(A, B, C)
        torch.cuda.synchronize()
    assert "tile_gemm: run" not in capfd.readouterr().err
