"""tile_partitioned_dense_amd -- tile-partitioned dense GEMM C = A.B on AMD
Instinct MI355X (gfx950).

Every output tile is exclusively owned by one workgroup, which reads A and B
as shared read-only views (the partition discipline of "GPU speed, without
leaving Rust's safety model", sections "Ownership crosses the launch
boundary" and "The useful boundary"). The compute runs in hand-written HIP
kernels behind a C ABI (``include/tile_gemm.h``); this package is the thin
Python binding over it.

The binding is imported lazily so that ``synth`` (the seeded input
generator) works without the compiled library. Any use of the GPU entry
points raises if ``libtile_gemm.so`` has not been built: there is no
fallback path.
"""

__all__ = ["tile_gemm_create", "tile_gemm_run", "tile_gemm_run_debug", "tile_gemm_run_epilogue",
           "tile_gemm_check_epilogue", "Act", "tile_gemm_destroy", "tile_gemm_run_mx",
           "tile_gemm_check_mx", "tile_gemm_plan_mx", "N_MX_CONFIGS", "MX_E4M3", "MX_E2M1", "VARIANT_MX",
           "tile_gemm_status_str", "tile_gemm_check_args", "tile_gemm_plan",
           "tile_gemm_tile_of", "TileGemm", "TileGemmError", "Status", "Dtype",
           "Strides", "Plan", "library_path", "load_library", "last_error_detail",
           "DEBUG_COUNT_WRITES", "DEBUG_COLLIDE", "DEBUG_FORCE_TILE",
           "DEBUG_FORCE_SKINNY", "DEBUG_FORCE_GRID", "DEBUG_ONE_TILE_PER_WG", "DEBUG_GROUP_M", "N_TILE_CONFIGS", "N_SKINNY_CONFIGS", "VARIANT_NONE", "VARIANT_TILE",
           "VARIANT_SKINNY"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
