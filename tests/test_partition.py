"""Host-side checks of the planner and the owned-tile map.

The output is partitioned into disjoint tiles before launch and each tile
has exactly one owning workgroup ("GPU speed, without leaving Rust's safety
model", section "Ownership crosses the launch boundary"). tile_gemm_tile_of
runs the same tile_of function the kernels run, compiled for the host, so
these tests check the device map itself: a bijection from tile numbers onto
the tile grid whose tiles cover C exactly once, and workgroup w owning tile
numbers w, w + grid, ...
"""

import itertools
import random

import pytest

import tile_partitioned_dense_amd as tg
from tile_partitioned_dense_amd import synth

CU = 256


def cover_check(M, N, K, bcol=False, cu=CU):
    plan = tg.tile_gemm_plan(M, N, K, bcol, cu)
    if M == 0 or N == 0:
        assert plan.variant == tg.VARIANT_NONE and plan.grid == 0 and plan.tiles == 0
        return plan
    check_grid(plan, cu)
    seen = set()
    area = 0
    for wg in range(plan.tiles):
        m0, n0, rows, cols = tg.tile_gemm_tile_of(plan, M, N, wg)
        assert (m0, n0) not in seen, f"tile ({m0},{n0}) owned twice"
        seen.add((m0, n0))
        assert 0 <= m0 < M and 0 <= n0 < N
        assert 0 < rows <= plan.bm and 0 < cols <= plan.bn
        assert m0 % plan.bm == 0 and n0 % plan.bn == 0
        assert rows == min(plan.bm, M - m0) and cols == min(plan.bn, N - n0)
        area += rows * cols
    # distinct grid-aligned tiles whose clipped areas sum to M*N cover C exactly
    assert area == M * N
    assert len(seen) == plan.tiles
    return plan


def check_grid(plan, cu):
    """Workgroup w owns tile numbers w, w + grid, ...: every tile has one owner
    by construction. One round of tiles gets one workgroup each; more rounds
    share the tiles out evenly, never needing more rounds than one tile per
    compute unit would, and keep a workgroup's tiles on one XCD."""
    T, G = plan.tiles, plan.grid
    assert 1 <= G <= T
    if plan.variant == tg.VARIANT_SKINNY or T <= cu:
        assert G == T
        return
    rounds = -(-T // cu)
    g0 = -(-T // rounds)
    g8 = -(-g0 // 8) * 8
    assert G == (g8 if g8 <= cu else g0)
    per_wg = [len(range(w, T, G)) for w in range(G)]
    assert max(per_wg) == rounds and max(per_wg) - min(per_wg) <= 1
    if G % 8 == 0:
        for w in range(0, G, max(1, G // 17)):
            assert all(t % 8 == w % 8 for t in range(w, T, G))


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_workload_partitions(name):
    w = synth.WORKLOADS[name]
    plan = cover_check(w.M, w.N, w.K, w.b_col_major)
    assert plan.grid >= 1


def test_expected_plans_for_workloads():
    W = synth.WORKLOADS
    p = tg.tile_gemm_plan(W["qkv_shard"].M, W["qkv_shard"].N, W["qkv_shard"].K, False, CU)
    assert (p.variant, p.bm, p.bn, p.tiles, p.grid) == (tg.VARIANT_TILE, 256, 160, 256, 256)
    # 256 x 224 tiles: 32 x 32 = 1024 tiles, 4 rounds of all 256 compute units
    # (256 x 256 tiles would be 4 rounds of 224)
    p = tg.tile_gemm_plan(8192, 7168, 8192, True, CU)
    assert (p.variant, p.bm, p.bn, p.tiles, p.grid) == (tg.VARIANT_TILE, 256, 224, 1024, 256)
    p = tg.tile_gemm_plan(4096, 4096, 4096, False, CU)
    assert (p.variant, p.bm, p.bn, p.tiles, p.grid) == (tg.VARIANT_TILE, 256, 256, 256, 256)
    p = tg.tile_gemm_plan(16, 28672, 8192, False, CU)
    assert p.variant == tg.VARIANT_SKINNY and p.k_split == 8 and p.bm == 16
    assert p.grid == p.tiles and p.grid * p.bn >= 28672 and (p.grid - 1) * p.bn < 28672


def test_few_rows_of_column_major_b_take_the_stream_kernel():
    """Column-major B, even K and M <= 64: the stream configurations (one
    tile row: 32 x 64 tiles with 256 K values per stage up to 32 rows, 64 x
    128 with 128 above); row-major B keeps the skinny kernel, 65 rows the
    tile kernel's other configurations."""
    for M in (1, 16, 17, 32):
        p = tg.tile_gemm_plan(M, 28672, 8192, True, CU)
        assert (p.variant, p.bm, p.bn, p.bk, p.tiles, p.grid) == (tg.VARIANT_TILE, 32, 64, 256, 448, 224)
    p = tg.tile_gemm_plan(64, 7168, 8192, True, CU)                 # few columns: 64 x 64
    assert (p.bm, p.bn, p.bk, p.tiles) == (64, 64, 128, 112)
    p = tg.tile_gemm_plan(64, 28672, 8192, True, CU)
    assert (p.bm, p.bn, p.bk, p.tiles, p.grid) == (64, 128, 128, 224, 224)
    assert tg.tile_gemm_plan(16, 28672, 8192, False, CU).variant == tg.VARIANT_SKINNY
    assert tg.tile_gemm_plan(65, 28672, 8192, True, CU).bk == 32
    assert tg.tile_gemm_plan(16, 28672, 8191, True, CU).variant == tg.VARIANT_SKINNY   # odd K


def test_persistent_grid_shares_tiles_evenly():
    # 8192^3: 1024 tiles of 256x256 -> 4 rounds of 256 workgroups;
    # 7168 x 6144: 28 x 24 = 672 tiles of 256x256 -> 3 rounds of 224
    p = tg.tile_gemm_plan(8192, 8192, 8192, False, CU)
    assert (p.bm, p.bn, p.tiles, p.grid) == (256, 256, 1024, 256)
    p = tg.tile_gemm_plan(7168, 6144, 8192, True, CU)
    assert (p.bm, p.bn, p.tiles, p.grid) == (256, 256, 672, 224)


def test_plan_is_a_pure_function_of_shape():
    a = tg.tile_gemm_plan(1000, 777, 333, False, CU).as_dict()
    for _ in range(3):
        assert tg.tile_gemm_plan(1000, 777, 333, False, CU).as_dict() == a


@pytest.mark.parametrize("M,N", [(1, 1), (65, 65), (257, 255), (1000, 1000), (17, 33),
                                 (64, 100000), (300, 7), (4096, 256), (8192, 1280),
                                 (2049, 4095), (63, 65), (65, 1), (512, 64 * 257)])
def test_edge_shape_partitions(M, N):
    for bcol in (False, True):
        cover_check(M, N, 64, bcol)


def test_random_shapes_partition():
    rng = random.Random(1234)
    for _ in range(60):
        M = rng.choice([rng.randint(1, 70), rng.randint(1, 3000)])
        N = rng.randint(1, 3000)
        cover_check(M, N, rng.randint(0, 500), rng.random() < 0.5)


@pytest.mark.parametrize("cu", [1, 7, 80, 256, 304])
def test_other_cu_counts(cu):
    cover_check(3000, 2000, 100, False, cu)
    cover_check(40, 5000, 100, False, cu)


def test_xcd_remap_keeps_neighbours_on_one_xcd():
    """Workgroups dispatched to one XCD (ids equal mod 8) get consecutive tile
    indices, so co-running tiles share panels."""
    plan = tg.tile_gemm_plan(8192, 7168, 8192, True, CU)
    assert plan.xcds == 8
    by_xcd = {}
    for wg in range(plan.tiles):
        m0, n0, _, _ = tg.tile_gemm_tile_of(plan, 8192, 7168, wg)
        by_xcd.setdefault(wg % 8, []).append((m0 // plan.bm, n0 // plan.bn))
    for x, tiles in by_xcd.items():
        first = tiles[:32]                       # one dispatch round of 32 CUs
        rows = {t[0] for t in first}
        cols = {t[1] for t in first}
        assert len(rows) * len(cols) <= 64, (x, rows, cols)


def test_plan_rejects_bad_input():
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_plan(-1, 4, 4)
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_plan(4, 4, 4, cu_count=0)
    plan = tg.tile_gemm_plan(512, 512, 64)
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_tile_of(plan, 512, 512, plan.tiles)


def _colliding_tile_of(plan, M, N, wg):
    """The negative-control map the debug entry point can force: workgroup 1
    takes workgroup 0's tile."""
    return tg.tile_gemm_tile_of(plan, M, N, 0 if wg == 1 else wg)


def test_negative_control_map_is_caught_by_cover_check():
    plan = tg.tile_gemm_plan(1024, 1024, 64)
    seen = set()
    dup = False
    for wg in range(plan.tiles):
        t = _colliding_tile_of(plan, 1024, 1024, wg)[:2]
        dup |= t in seen
        seen.add(t)
    assert dup and len(seen) == plan.tiles - 1


@pytest.mark.parametrize("M,N", [(8192, 7168), (8192, 1280), (1000, 3000), (300, 257)])
@pytest.mark.parametrize("group_m", [1, 2, 3, 5, 8, 13, 63])
def test_tile_of_is_a_bijection_for_any_raster_group(M, N, group_m):
    """The debug raster-group override (TILE_GEMM_DEBUG_GROUP_M) only changes
    the order of tiles: for every height the map stays a bijection."""
    plan = tg.tile_gemm_plan(M, N, 4096, False, CU)
    plan.group_m = min(group_m, plan.tiles_m)
    seen = set()
    for wg in range(plan.tiles):
        m0, n0, rows, cols = tg.tile_gemm_tile_of(plan, M, N, wg)
        seen.add((m0, n0))
    assert len(seen) == plan.tiles


def test_rate_tool_reads_the_configuration_table():
    """The configuration-rate tool (tile_partitioned_dense_amd/rate_configs.py)
    reads the planner's table from plan.hpp: it must see every entry with the
    struct's defaults applied."""
    from tile_partitioned_dense_amd import build, rate_configs
    t = rate_configs.config_table()
    assert len(t) == build.N_TILE_CONFIGS
    assert t[0] == dict(bm=256, bn=256, wm=2, wn=2, stages=4, eff=0.94, ks=1, eff1=0.0, occ=1, sb=0,
                        mi=32, bk=32)
    assert t[5]["eff1"] == 0.59 and t[5]["occ"] == 2
    assert t[14]["sb"] == 512 and t[14]["ks"] == 2
    assert t[17]["mi"] == 16 and t[17]["bk"] == 32
    assert t[24]["mi"] == 16 and t[24]["bk"] == 64
