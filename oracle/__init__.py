"""CPU oracle for the tile-partitioned dense product C = A.B.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The GPU library
and its Python binding never import it, and it imports nothing from them: the
two sides share no code, tables or helpers. The only thing both sides see is
the seeded input generator (``tile_partitioned_dense_amd.synth``), which holds
no arithmetic of the product itself.

Contents
--------
* ``gemm`` / ``gemm_at``  -- the plain fp64 triple loop in C
  (``gemm_oracle.c``): full product, or selected elements one at a time.
* ``gemm_blas``           -- the same definition evaluated by a library fp64
  matrix product (a library primitive used as one step), for full-size
  comparisons the triple loop would take minutes for. Exact for
  integer-valued inputs; otherwise within K*2^-53*D of the exact sum.
* ``bf16_to_f64`` / ``rne_bf16`` -- the oracle's own bf16 decode and
  round-to-nearest-even encode (directly from fp64, no double rounding).
* ``check_f32`` / ``check_bf16`` / ``check_exact`` -- the acceptance rules.
* ``epilogue`` / ``check_epilogue`` -- the fused epilogue act(C + bias) in
  fp64 and its acceptance rule (``fused_epilogue.py``); ``swiglu`` /
  ``check_swiglu`` -- SiLU(gate) * up on a merged gate+up product.
* ``mx`` -- the microscaled (MXFP8 / MXFP4) product: E4M3, E2M1 and E8M0
  decoding and the scaled sum in fp64 (``mx.py``); its results are checked
  with ``check_f32`` / ``check_bf16`` like the bf16 product's.

Parity pins (tests/test_oracle_pins.py) tie every function here to
something other than itself: exact rational brute force, identity and
permutation closed forms, integer exactness against an int64 loop, the
ones/diagonal closed forms, hand-derived bf16 rounding cases and planted
mistakes that each pin must catch.
"""

from .reference import (  # noqa: F401
    build,
    lib_path,
    open_library,
    max_threads,
    gemm,
    gemm_at,
    gemm_blas,
)
from .numerics import (  # noqa: F401
    bf16_to_f64,
    rne_bf16,
    check_f32,
    check_bf16,
    check_exact,
    CheckReport,
)
from .fused_epilogue import (  # noqa: F401
    ACTS,
    act_f64,
    epilogue,
    epilogue_bound,
    check_epilogue,
    swiglu,
    swiglu_bound,
    check_swiglu,
)
from . import mx  # noqa: F401,E402
