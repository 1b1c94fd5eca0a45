"""Host-only checks of the C ABI: the library loads and exports every entry
point the header declares, argument checks return the documented codes, and
create refuses a machine without a gfx950. No compute is launched here."""

import ctypes
import os
import re

import pytest

import tile_partitioned_dense_amd as tg
from tile_partitioned_dense_amd.binding import Dtype, Status, Strides

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tile_gemm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(tile_gemm_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = tg.load_library()
    names = declared_functions()
    assert len(names) >= 9, names
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings():
    for s in Status:
        txt = tg.tile_gemm_status_str(s)
        assert isinstance(txt, str) and txt
    assert tg.tile_gemm_status_str(99) == "unknown status"


def test_create_without_gfx950_fails_cleanly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible; covered by the GPU tests")
    lib = tg.load_library()
    h = ctypes.c_void_p(1234)
    st = lib.tile_gemm_create(ctypes.byref(h), 0)
    assert st == Status.ERR_DEVICE
    assert h.value is None
    assert "device" in tg.last_error_detail()
    assert lib.tile_gemm_create(None, 0) == Status.ERR_NULL_ARG


def test_destroy_null_is_ok_and_run_null_handle():
    lib = tg.load_library()
    assert lib.tile_gemm_destroy(None) == Status.OK
    s = Strides(8, 1, 8, 1, 8, 1)
    st = lib.tile_gemm_run(None, 16, 16, 4096, 4, 4, 4, ctypes.byref(s), 0, None)
    assert st == Status.ERR_NULL_ARG


# --- argument checks (pointers are plain aligned integers; nothing is touched)
A0, B0, C0 = 0x100000, 0x200000, 0x300000


def chk(A=A0, B=B0, C=C0, M=64, N=64, K=64, s=(64, 1, 64, 1, 64, 1), dtype=Dtype.BF16_TO_F32):
    return tg.tile_gemm_check_args(A, B, C, M, N, K, s, dtype)


def test_check_args_ok_layouts():
    assert chk() == Status.OK
    assert chk(s=(64, 1, 1, 64, 64, 1)) == Status.OK           # column-major B
    assert chk(s=(72, 1, 80, 1, 96, 1)) == Status.OK           # padded leading dims
    assert chk(dtype=Dtype.BF16_TO_BF16) == Status.OK
    assert chk(M=0, A=0, B=0, C=0) == Status.OK                # empty: pointers unchecked
    assert chk(N=0, A=0, B=0, C=0) == Status.OK
    assert chk(K=0, s=(0, 1, 64, 1, 64, 1)) == Status.OK       # K = 0 writes zeros


@pytest.mark.parametrize("kw,want", [
    (dict(dtype=7), Status.ERR_DTYPE),
    (dict(M=-1), Status.ERR_BAD_SHAPE),
    (dict(K=-3), Status.ERR_BAD_SHAPE),
    (dict(N=1 << 31), Status.ERR_BAD_SHAPE),
    (dict(A=0), Status.ERR_NULL_ARG),
    (dict(B=0), Status.ERR_NULL_ARG),
    (dict(C=0), Status.ERR_NULL_ARG),
    (dict(s=(64, 2, 64, 1, 64, 1)), Status.ERR_BAD_STRIDE),    # A not K-contiguous
    (dict(s=(32, 1, 64, 1, 64, 1)), Status.ERR_BAD_STRIDE),    # a_m < K
    (dict(s=(64, 1, 32, 1, 64, 1)), Status.ERR_BAD_STRIDE),    # b_k < N
    (dict(s=(64, 1, 1, 32, 64, 1)), Status.ERR_BAD_STRIDE),    # b_n < K
    (dict(s=(64, 1, 64, 2, 64, 1)), Status.ERR_BAD_STRIDE),    # B neither layout
    (dict(s=(64, 1, 64, 1, 64, 2)), Status.ERR_BAD_STRIDE),    # C not row-major
    (dict(s=(64, 1, 64, 1, 32, 1)), Status.ERR_BAD_STRIDE),    # c_m < N
    (dict(A=A0 + 2), Status.ERR_MISALIGNED),
    (dict(B=B0 + 8), Status.ERR_MISALIGNED),
    (dict(C=C0 + 4), Status.ERR_MISALIGNED),
    (dict(K=60, s=(60, 1, 64, 1, 64, 1)), Status.ERR_MISALIGNED),   # a_m*2 not /16
    (dict(N=60, s=(64, 1, 60, 1, 64, 1)), Status.ERR_MISALIGNED),   # b_k*2 not /16
    (dict(N=62, s=(64, 1, 64, 1, 62, 1)), Status.ERR_MISALIGNED),   # fp32 c_m*4 not /16
    (dict(C=A0 + 1024), Status.ERR_ALIAS),                           # C inside A
    (dict(C=B0 - 1024), Status.ERR_ALIAS),                           # C runs into B
    (dict(s=None), Status.ERR_NULL_ARG),
    (dict(M=70000, K=32768, s=(32768, 1, 64, 1, 64, 1)), Status.ERR_BAD_SHAPE),   # A >= 4 GiB
    (dict(N=70000, K=32768, s=(32768, 1, 1, 32768, 70000, 1)), Status.ERR_BAD_SHAPE),  # B >= 4 GiB
])
def test_check_args_errors(kw, want):
    if "s" in kw and kw["s"] is None:
        lib = tg.load_library()
        st = lib.tile_gemm_check_args(A0, B0, C0, 64, 64, 64, None, 0)
        assert st == want
        return
    assert chk(**kw) == want
    assert tg.last_error_detail(), "a failed check names its argument"


def test_bf16_output_alignment_rule():
    # c_m = 60 bf16 elements = 120 bytes, not a multiple of 16
    assert chk(N=60, s=(64, 1, 64, 1, 60, 1), dtype=Dtype.BF16_TO_BF16) == Status.ERR_MISALIGNED
    # c_m = 56 bf16 elements = 112 bytes: fine; fp32 the same c_m = 224 bytes: fine
    assert chk(N=56, s=(64, 1, 64, 1, 56, 1), dtype=Dtype.BF16_TO_BF16) == Status.OK


def test_alias_adjacent_is_not_overlap():
    # A occupies [A0, A0 + 2*(63*64 + 64)); C starting exactly at its end is fine
    a_end = A0 + 2 * (63 * 64 + 64)
    assert chk(C=a_end) == Status.OK
    assert chk(C=a_end - 16) == Status.ERR_ALIAS


def test_config_counts_match_the_compiled_tables():
    """The Python-side counts of compiled configurations (build loop, forced
    configuration flags) equal the table sizes in plan.hpp."""
    from tile_partitioned_dense_amd import binding, build
    plan_src = open(os.path.join(ROOT, "tile_partitioned_dense_amd", "csrc", "plan.hpp")).read()
    n_tile = int(re.search(r"kNumTileConfigs\s*=\s*(\d+)", plan_src).group(1))
    n_skinny = int(re.search(r"kNumSkinnyConfigs\s*=\s*(\d+)", plan_src).group(1))
    assert binding.N_TILE_CONFIGS == build.N_TILE_CONFIGS == n_tile
    assert binding.N_SKINNY_CONFIGS == build.N_SKINNY_CONFIGS == n_skinny
    table = re.search(r"kTileConfigs\[kNumTileConfigs\]\s*=\s*\{(.*?)\n\};", plan_src, re.S).group(1)
    assert len(re.findall(r"^\s*\{\d+,", table, re.M)) == n_tile


# --- fused epilogue argument checks
def chk_epi(bias=0x400000, act=0, C=C0, M=64, N=64, s=(64, 1, 64, 1, 64, 1), dtype=Dtype.BF16_TO_F32):
    return tg.tile_gemm_check_epilogue(C, M, N, s, dtype, bias, act)


def test_check_epilogue():
    from tile_partitioned_dense_amd.binding import Act
    for a in Act:
        assert chk_epi(act=a) == Status.OK
        assert chk_epi(bias=None, act=a) == Status.OK          # bias is optional
    assert chk_epi(act=6) == Status.ERR_EPILOGUE
    assert chk_epi(act=-1) == Status.ERR_EPILOGUE
    assert "activation" in tg.last_error_detail()
    assert chk_epi(bias=0x400004) == Status.ERR_MISALIGNED
    assert chk_epi(bias=C0 + 64) == Status.ERR_ALIAS            # bias inside C
    # fp32 C of 64 x 64 ends at C0 + 16384: a bias right there is fine, 16 bytes earlier is not
    assert chk_epi(bias=C0 + 4 * 64 * 64) == Status.OK
    assert chk_epi(bias=C0 + 4 * 64 * 64 - 16) == Status.ERR_ALIAS
    # bf16 C is half as long
    assert chk_epi(bias=C0 + 2 * 64 * 64, dtype=Dtype.BF16_TO_BF16) == Status.OK
    assert chk_epi(bias=C0 - 4 * 64) == Status.OK               # bias ends where C starts
    assert chk_epi(bias=C0 - 4 * 64 + 16) == Status.ERR_ALIAS
    assert chk_epi(M=0, bias=0x400004) == Status.OK             # empty output: nothing read


def test_run_epilogue_null_handle_and_bad_act():
    lib = tg.load_library()
    s = Strides(64, 1, 64, 1, 64, 1)
    assert lib.tile_gemm_run_epilogue(None, A0, B0, C0, 64, 64, 64, ctypes.byref(s), 0, None, 0,
                                      None) == Status.ERR_NULL_ARG


def test_check_swiglu_widths():
    from tile_partitioned_dense_amd.binding import Act
    # N counts gate + up columns and must be a multiple of 16; C is M x N/2
    assert chk_epi(act=Act.SWIGLU, N=64) == Status.OK
    assert chk_epi(act=Act.SWIGLU, N=72, s=(64, 1, 72, 1, 72, 1)) == Status.ERR_BAD_SHAPE
    # the bias (N values) may sit right after C's M x N/2 fp32 elements
    assert chk_epi(act=Act.SWIGLU, bias=C0 + 4 * (63 * 64 + 32)) == Status.OK
    assert chk_epi(act=Act.SWIGLU, bias=C0 + 4 * (63 * 64 + 32) - 16) == Status.ERR_ALIAS


# --- MX argument checks
SA0, SB0 = 0x500000, 0x600000


def chk_mx(A=A0, B=B0, C=C0, M=64, N=64, K=128, s=(128, 1, 1, 128, 64, 1), sa=SA0, sb=SB0,
           ls=4, dtype=Dtype.BF16_TO_F32, bias=None, act=0, fmt=0):
    return tg.tile_gemm_check_mx(A, B, C, M, N, K, s, sa, sb, ls, dtype, bias, act, fmt)


@pytest.mark.parametrize("kw,want", [
    (dict(), Status.OK),
    (dict(K=0, A=0, B=0, sa=0, sb=0), Status.OK),
    (dict(M=0), Status.OK),
    (dict(K=96, s=(128, 1, 1, 128, 64, 1)), Status.ERR_BAD_SHAPE),      # K % 64
    (dict(fmt=2), Status.ERR_DTYPE),
    (dict(fmt=1), Status.OK),                                           # E2M1: K = 128 fits
    (dict(fmt=1, K=64, s=(64, 1, 1, 64, 64, 1), ls=4), Status.ERR_BAD_SHAPE),   # E2M1 K % 128
    (dict(fmt=1, s=(48, 1, 1, 64, 64, 1)), Status.ERR_BAD_STRIDE),      # E2M1 a_m < K/2 bytes
    (dict(dtype=5), Status.ERR_DTYPE),
    (dict(sa=0), Status.ERR_NULL_ARG),
    (dict(s=(128, 1, 128, 1, 64, 1)), Status.ERR_BAD_STRIDE),           # B not K-contiguous
    (dict(s=(64, 1, 1, 128, 64, 1)), Status.ERR_BAD_STRIDE),            # a_m < K
    (dict(ls=2), Status.ERR_BAD_STRIDE),                                # ls not a multiple of 4
    (dict(ls=0), Status.ERR_BAD_STRIDE),                                # ls < K/32
    (dict(A=A0 + 8), Status.ERR_MISALIGNED),
    (dict(sa=SA0 + 2), Status.ERR_MISALIGNED),
    (dict(s=(136, 1, 1, 128, 64, 1)), Status.ERR_MISALIGNED),           # a_m not /16
    (dict(C=SA0 + 64), Status.ERR_ALIAS),                               # C over a_scale
    (dict(act=5), Status.ERR_EPILOGUE),                                 # no SiLU(gate)*up
    (dict(bias=0x700004, act=1), Status.ERR_MISALIGNED),
])
def test_check_mx(kw, want):
    assert chk_mx(**kw) == want, tg.last_error_detail()


def test_mx_plan():
    """The MX MLP shard, both formats: 256 x 224 tiles on 16x16x128 blocks
    (configuration 7), 1024 tiles in four rounds of all 256 compute units.
    At 4096^3 the 256 x 256 tiles of the 128-byte-row 32x32x64 kernel
    (configuration 6) fill one round. An unknown format is refused."""
    for fmt in (tg.MX_E4M3, tg.MX_E2M1):
        p = tg.tile_gemm_plan_mx(8192, 7168, 8192, fmt)
        assert p.variant == tg.VARIANT_MX and p.config == 7 and (p.bm, p.bn, p.bk) == (256, 224, 128)
        assert p.tiles == 32 * 32 and p.grid == 256
        p = tg.tile_gemm_plan_mx(4096, 4096, 4096, fmt)
        assert p.config == 6 and (p.bm, p.bn, p.tiles) == (256, 256, 256)
    # a K that is not a multiple of 128 keeps E4M3 off the 16x16x128 blocks
    assert tg.tile_gemm_plan_mx(8192, 7168, 8192 + 64, tg.MX_E4M3).config == 6
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_plan_mx(8192, 7168, 8192, 7)


def test_mx_plan_few_rows_take_the_stream_kernel():
    """Outputs of up to 64 rows stream B (one tile row of 32 or 64 rows x 128
    columns, 256 bytes of K per stage); from 65 rows the tile kernel's
    configurations."""
    for M, cfg, bm in ((1, 3, 32), (16, 3, 32), (17, 3, 32), (32, 3, 32), (33, 4, 64), (64, 4, 64)):
        p = tg.tile_gemm_plan_mx(M, 28672, 8192)
        assert (p.variant, p.config, p.bm, p.bn, p.bk) == (tg.VARIANT_MX, cfg, bm, 128, 256), M
        assert p.tiles == 28672 // p.bn and p.grid == 224
    assert tg.tile_gemm_plan_mx(65, 28672, 8192).bk == 64
    # few columns: 64-column tiles with 512-byte stages keep more compute units busy
    p = tg.tile_gemm_plan_mx(16, 7168, 8192)
    assert (p.config, p.bm, p.bn, p.bk, p.tiles) == (5, 32, 64, 512, 112)


def test_smoke_shape_passes_the_argument_checks():
    """smoke() hands contiguous operands of SMOKE_SHAPE to the library, so that
    shape must satisfy its alignment rules for both B layouts it could use."""
    import __graft_entry__ as ge
    M, N, K = ge.SMOKE_SHAPE
    for dt in (Dtype.BF16_TO_F32, Dtype.BF16_TO_BF16):
        assert chk(M=M, N=N, K=K, s=(K, 1, N, 1, N, 1), dtype=dt) == Status.OK, tg.last_error_detail()


# --- strides that would overflow the span arithmetic (each was accepted before
# the leading dimensions were bounded and the spans computed with checks)
@pytest.mark.parametrize("kw", [
    dict(M=5, s=(1 << 62, 1, 64, 1, 64, 1)),                 # a_m = 2^62
    dict(M=5, s=(1 << 31, 1, 64, 1, 64, 1)),                 # a_m = 2^31
    dict(s=(64, 1, 1 << 62, 1, 64, 1)),                      # row-major b_k = 2^62
    dict(s=(64, 1, 1, 1 << 62, 64, 1)),                      # column-major b_n = 2^62
    dict(s=(64, 1, 64, 1, 1 << 61, 1)),                      # c_m = 2^61
    dict(s=(64, 1, 64, 1, 1 << 62, 1), C=A0 - 0x1000),       # c_m = 2^62, C just below A
    dict(K=0, s=(0, 1, 64, 1, 1 << 62, 1)),                  # K = 0 still checks C
])
def test_check_args_refuses_huge_strides(kw):
    st = chk(**kw)
    assert st in (Status.ERR_BAD_STRIDE, Status.ERR_BAD_SHAPE), (kw, st)
    assert tg.last_error_detail()


@pytest.mark.parametrize("kw", [
    dict(s=(1 << 62, 1, 1, 128, 64, 1)),                     # a_m
    dict(s=(128, 1, 1, 1 << 62, 64, 1)),                     # b_n
    dict(s=(128, 1, 1, 128, 1 << 61, 1)),                    # c_m
    dict(ls=1 << 40),                                        # scale_stride
    dict(ls=(1 << 31) // 64 // 4 * 4 * 4),                   # (M + 256) * ls >= 2^31
])
def test_check_mx_refuses_huge_strides(kw):
    st = chk_mx(**kw)
    assert st in (Status.ERR_BAD_STRIDE, Status.ERR_BAD_SHAPE), (kw, st)


# --- the binding's own checks of torch tensors (the C ABI sees raw pointers
# only, so a host tensor, a wrong dtype or a short bias must stop here)
def _bf16(*shape):
    import torch
    return torch.zeros(*shape, dtype=torch.bfloat16)


def test_binding_refuses_host_tensors():
    import torch
    A, B = _bf16(64, 64), _bf16(64, 64)
    C = torch.zeros(64, 64, dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        tg.tile_gemm_run(None, A, B, C)
    with pytest.raises(ValueError, match="GPU"):
        tg.tile_gemm_run_epilogue(None, A, B, C)


def test_binding_refuses_dtype_mismatch():
    import torch
    A, B = _bf16(64, 64), _bf16(64, 64)
    C = _bf16(64, 64)
    with pytest.raises(TypeError, match="does not match"):
        tg.tile_gemm_run(None, A, B, C, dtype=Dtype.BF16_TO_F32)
    with pytest.raises(TypeError, match="bfloat16"):
        tg.tile_gemm_run(None, A.float(), B, C)
    with pytest.raises(TypeError, match="float32 or bfloat16"):
        tg.tile_gemm_run(None, A, B, C.to(torch.float16))


@pytest.mark.parametrize("bias_kw,err", [
    (dict(n=64, dtype="bfloat16"), TypeError),
    (dict(n=63, dtype="float32"), ValueError),
    (dict(n=128, dtype="float32", step=2), ValueError),
])
def test_binding_refuses_bad_bias(bias_kw, err):
    import torch
    A, B = _bf16(64, 64), _bf16(64, 64)
    C = torch.zeros(64, 64, dtype=torch.float32)
    bias = torch.zeros(bias_kw["n"], dtype=getattr(torch, bias_kw["dtype"]))
    if bias_kw.get("step"):
        bias = bias[::bias_kw["step"]]
    with pytest.raises(err):
        tg.tile_gemm_run_epilogue(None, A, B, C, bias=bias)


def test_binding_refuses_mixed_pointer_kinds():
    with pytest.raises(TypeError, match="all torch tensors or all raw pointers"):
        tg.tile_gemm_run(None, _bf16(8, 8), 0x1000, 0x2000, 8, 8, 8, (8, 1, 8, 1, 8, 1), 0)


def test_binding_mx_scale_stride_of_single_rows():
    """A single-row scale array's row stride is meaningless (numpy and torch
    keep whatever the parent had); the binding passes the other array's."""
    import numpy as np
    import torch
    from tile_partitioned_dense_amd.binding import _mx_operands
    a = torch.zeros(1, 64, dtype=torch.uint8)
    bt = torch.zeros(64, 64, dtype=torch.uint8)
    c = torch.zeros(1, 64, dtype=torch.float32)
    sa = torch.from_numpy(np.ascontiguousarray(np.zeros((1, 5), np.uint8)[:, :4]))
    sb = torch.zeros(64, 4, dtype=torch.uint8)
    assert sa.stride(0) != sb.stride(0) or True
    M, N, K, s, ls, dt = _mx_operands(a, bt, c, sa, sb, tg.MX_E2M1)
    assert (M, N, K, ls) == (1, 64, 128, 4)
    with pytest.raises(ValueError, match="common stride"):
        _mx_operands(torch.zeros(2, 64, dtype=torch.uint8), bt, torch.zeros(2, 64), torch.zeros(2, 8, dtype=torch.uint8)[:, :4], sb, tg.MX_E2M1)
