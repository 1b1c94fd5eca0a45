"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Acceptance, per element: fp32 output within 1e-5 * (|A|.|B|)_ij of the
oracle; bf16 output inside the RNE bracket of that interval; integer-valued
inputs exactly equal. Every output starts as a NaN sentinel (padding columns
included), so a missed element or a write outside the owned region shows.
"""

import numpy as np
import pytest

import oracle
import tile_partitioned_dense_amd as tg
from tile_partitioned_dense_amd import synth

from gpu_helpers import Case, check, host_out, stream_tile_configs, tile_config_table, workload_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    with tg.TileGemm(0) as gg:
        yield gg


def _run(g, case, dtype, flags=0, counts=None):
    store, C = case.out(dtype)
    if flags:
        g.run_debug(case.A_dev, case.B_dev, C, counts=counts, flags=flags)
    else:
        g(case.A_dev, case.B_dev, C)
    torch.cuda.synchronize()
    return store, C


def _assert_padding_untouched(store, N):
    pad = store[:, N:]
    if pad.numel():
        assert torch.isnan(pad.float()).all(), "a store landed outside the owned columns"


def _parity(g, case, dtype, flags=0, integer=False):
    store, C = _run(g, case, dtype, flags)
    out = host_out(C)
    Cr, Dr = case.ref()
    rep = check(out, Cr, Dr, dtype == torch.bfloat16, integer)
    assert rep.ok, f"{case.M}x{case.N}x{case.K} bcol={case.bcol} {dtype}: {rep}"
    _assert_padding_untouched(store, case.N)
    return out


# ------------------------------------------------ every compiled configuration

def tile_shape(cfg):
    bm, bn = tile_config_table()[cfg][:2]
    return 2 * bm + 37, 2 * bn + 19     # several tiles plus a ragged edge in M and N


@pytest.mark.parametrize("cfg", range(tg.N_TILE_CONFIGS))
@pytest.mark.parametrize("bcol", [False, True], ids=["Brow", "Bcol"])
def test_tile_configs(g, cfg, bcol):
    if cfg in stream_tile_configs() and not bcol:
        pytest.skip("stream configurations take a column-major B (rejection: test_gpu_stream)")
    M, N = tile_shape(cfg)
    print(f"[tile cfg {cfg} bcol={bcol} {M}x{N}x200]", flush=True)
    case = Case(M, N, 200, bcol, seed=cfg, pad=8)     # K = 3 slabs + a partial one
    for dt in (torch.float32, torch.bfloat16):
        _parity(g, case, dt, flags=tg.DEBUG_FORCE_TILE(cfg))


@pytest.mark.parametrize("cfg", range(tg.N_TILE_CONFIGS))
def test_tile_configs_integer_k_tail(g, cfg):
    """Integer data, K not a multiple of 8: exact, and the K tail is masked
    (the stream configurations, column-major B only, take an even K: 130)."""
    M, N = tile_shape(cfg)
    stream = cfg in stream_tile_configs()
    K = 130 if stream else 131
    print(f"[tile int cfg {cfg} {M}x{N}x{K}]", flush=True)
    for bcol in ((True,) if stream else (False, True)):
        case = Case(M, N, K, bcol, dist="int3", seed=10 + cfg)
        for dt in (torch.float32, torch.bfloat16):
            _parity(g, case, dt, flags=tg.DEBUG_FORCE_TILE(cfg), integer=True)


@pytest.mark.parametrize("cfg", [c for c in range(tg.N_TILE_CONFIGS) if c not in stream_tile_configs()])
def test_tile_configs_odd_n_whole_slabs(g, cfg):
    """Row-major B, odd N and K a multiple of 32, integer data, exact. B's last
    value (K - 1, N - 1) then shares a dword with the first padding element;
    a buffer load zeroes a dword that straddles the end of its resource, so
    that slab must not go through the DMA path (every term of column N - 1
    would lose A[:, K - 1] * B[K - 1, N - 1])."""
    M, N = tile_shape(cfg)          # N = 2 bn + 19: odd
    assert N % 2 == 1
    for K in (256, 64):
        print(f"[tile odd-N cfg {cfg} {M}x{N}x{K}]", flush=True)
        case = Case(M, N, K, False, dist="int3", seed=40 + cfg)
        for dt in (torch.float32, torch.bfloat16):
            _parity(g, case, dt, flags=tg.DEBUG_FORCE_TILE(cfg), integer=True)


@pytest.mark.parametrize("M,N,K", [(300, 257, 256), (40, 33, 64), (2000, 1001, 512)])
def test_planner_odd_n_whole_slabs(g, M, N, K):
    print(f"[planner odd-N {M}x{N}x{K}]", flush=True)
    case = Case(M, N, K, False, dist="int3", seed=M + N)
    for dt in (torch.float32, torch.bfloat16):
        _parity(g, case, dt, integer=True)
    ncase = Case(M, N, K, False, seed=M + N + 1)
    _parity(g, ncase, torch.float32)


SKINNY_MG = {0: 1, 1: 1, 2: 2, 3: 2, 4: 4, 5: 4}


@pytest.mark.parametrize("cfg", range(tg.N_SKINNY_CONFIGS))
@pytest.mark.parametrize("bcol", [False, True], ids=["Brow", "Bcol"])
def test_skinny_configs(g, cfg, bcol):
    mg = SKINNY_MG[cfg]
    for M in sorted({1, 5, 16 * mg - 3, 16 * mg}):
        N, K = 16 * 8 * 5 + 13, 8 * 32 * 3 + 24 + 5      # ragged N; K tail inside a 32-block
        print(f"[skinny cfg {cfg} bcol={bcol} {M}x{N}x{K}]", flush=True)
        case = Case(M, N, K, bcol, seed=20 + cfg, pad=8)
        for dt in (torch.float32, torch.bfloat16):
            _parity(g, case, dt, flags=tg.DEBUG_FORCE_SKINNY(cfg))
        icase = Case(M, N, K, bcol, dist="int3", seed=30 + cfg)
        _parity(g, icase, torch.float32, flags=tg.DEBUG_FORCE_SKINNY(cfg), integer=True)


# ------------------------------------------------------------- planner path

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (17, 33, 65), (257, 257, 257), (1000, 1000, 1000),
                                   (65, 300, 64), (64, 1, 9), (3, 5000, 300), (300, 7, 48),
                                   (4096, 256, 512), (130, 130, 0)])
@pytest.mark.parametrize("bcol", [False, True], ids=["Brow", "Bcol"])
def test_edge_shapes(g, M, N, K, bcol):
    print(f"[edge {M}x{N}x{K} bcol={bcol}]", flush=True)
    case = Case(M, N, K, bcol, seed=M + N + K)
    for dt in (torch.float32, torch.bfloat16):
        _parity(g, case, dt)     # K == 0: D == 0, so the check demands exact zeros
    icase = Case(M, N, K, bcol, dist="int3", seed=M + N + K + 1)
    _parity(g, icase, torch.float32, integer=True)


def test_empty_is_noop(g):
    A = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(64, 64, dtype=torch.bfloat16, device="cuda")
    C = torch.zeros(0, 64, dtype=torch.float32, device="cuda")
    assert g(A, B, C) == tg.Status.OK


# ----------------------------------------------------------- full workloads

WORKLOADS = sorted(synth.WORKLOADS)


def _run_workload(g, A, B, w, dtype):
    C = torch.full((w.M, w.N), float("nan"), dtype=dtype, device="cuda")
    g(A, B, C)
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("name", WORKLOADS)
def test_workload_parity(g, name):
    w, ops, A, B = workload_case(name)
    print(f"[workload {name} {w.M}x{w.N}x{w.K}]", flush=True)
    outs = {dt: host_out(_run_workload(g, A, B, w, dt))
            for dt in (torch.float32, torch.bfloat16)}
    # every element against the plain fp64 triple loop (ascending k per element)
    Cr, Dr = oracle.gemm(ops.A, ops.B)
    for dt, out in outs.items():
        rep = check(out, Cr, Dr, dt == torch.bfloat16)
        assert rep.ok, f"{name} {dt}: {rep}"
        print(f"  {dt}: max |g-C|/D = {rep.max_ratio:.3e}", flush=True)


@pytest.mark.parametrize("name", WORKLOADS)
def test_workload_integer_exact(g, name):
    w, ops, A, B = workload_case(name, integer=True)
    print(f"[workload int {name}]", flush=True)
    Cr, _ = oracle.gemm_blas(ops.A, ops.B, want_d=False)
    for dt in (torch.float32, torch.bfloat16):
        out = host_out(_run_workload(g, A, B, w, dt))
        rep = oracle.check_exact(out, Cr, dt == torch.bfloat16)
        assert rep.ok, f"{name} {dt}: {rep}"


# The decode / tall-skinny sweep: decode batches of 1-64 rows against the
# widest weight of the gate+up projection, in both B layouts, and the
# tall-skinny (4096, 256, 4096) shape; every element against the plain loop.
SWEEP = [(M, 28672, 8192, bcol) for M in (1, 8, 32, 64) for bcol in (False, True)] + \
        [(4096, 256, 4096, False), (4096, 256, 4096, True)]


class _Rows:
    """The first M rows of a larger case's A against its B (the decode shapes of
    one width share their weight matrix, which takes seconds to draw)."""

    def __init__(self, base, M):
        self.base, self.M, self.N, self.K, self.bcol = base, M, base.N, base.K, base.bcol
        self.A, self.B = base.A[:M], base.B
        self.A_dev, self.B_dev = base.A_dev[:M], base.B_dev
        self.pad, self.device, self._ref = base.pad, base.device, None

    def out(self, dtype, fill=float("nan")):
        return Case.out(self, dtype, fill)

    def ref(self):
        if self._ref is None:
            self._ref = oracle.gemm(self.A, self.B)
        return self._ref


@pytest.fixture(scope="module")
def sweep_bases():
    cache = {}

    def get(M, N, K, bcol, dist):
        rows = 64 if M <= 64 else M
        key = (rows, N, K, bcol, dist)
        if key not in cache:
            cache[key] = Case(rows, N, K, bcol, dist=dist, seed=3 * N + K + (7 if dist == "int3" else 0),
                              b_scale=1.0 if dist == "int3" else K ** -0.5, pad=8)
        return _Rows(cache[key], M)
    yield get
    cache.clear()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M,N,K,bcol", SWEEP)
def test_sweep_shapes_parity(g, sweep_bases, M, N, K, bcol):
    print(f"[sweep {M}x{N}x{K} bcol={bcol}]", flush=True)
    case = sweep_bases(M, N, K, bcol, "normal")
    for dt in (torch.float32, torch.bfloat16):
        _parity(g, case, dt)
    icase = sweep_bases(M, N, K, bcol, "int3")
    _parity(g, icase, torch.bfloat16, integer=True)


def test_bf16_output_is_rne_of_fp32_output(g):
    """One shape in both output modes: same plan, same K order, so the bf16
    result is the round-to-nearest-even of the fp32 result, bitwise."""
    w, ops, A, B = workload_case("square4096")
    f32 = host_out(_run_workload(g, A, B, w, torch.float32))
    b16 = host_out(_run_workload(g, A, B, w, torch.bfloat16))
    assert np.array_equal(b16, oracle.rne_bf16(f32.astype(np.float64)))
