"""Thin ctypes binding of libtile_gemm.so (include/tile_gemm.h).

Argument marshalling only: torch supplies device memory and the current
stream; every step of the product runs in the library's HIP kernels. There is
no fallback: if the library is missing, loading it raises.
"""

from __future__ import annotations

import ctypes
import enum
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libtile_gemm.so")
_lib = None


class Status(enum.IntEnum):
    OK = 0
    ERR_NULL_ARG = 1
    ERR_BAD_SHAPE = 2
    ERR_BAD_STRIDE = 3
    ERR_MISALIGNED = 4
    ERR_ALIAS = 5
    ERR_DTYPE = 6
    ERR_DEVICE = 7
    ERR_HIP = 8
    ERR_EPILOGUE = 9


class Dtype(enum.IntEnum):
    BF16_TO_F32 = 0
    BF16_TO_BF16 = 1


class Act(enum.IntEnum):
    NONE = 0
    RELU = 1
    SIGMOID = 2
    TANH = 3
    SILU = 4
    SWIGLU = 5


DEBUG_COUNT_WRITES = 1
DEBUG_COLLIDE = 2


def DEBUG_FORCE_TILE(c: int) -> int:
    return ((c + 1) & 0xFF) << 8


def DEBUG_FORCE_SKINNY(c: int) -> int:
    return ((c + 1) & 0xFF) << 16


def DEBUG_FORCE_GRID(g: int) -> int:
    return (g & 0x7F) << 24


DEBUG_ONE_TILE_PER_WG = 0x7F << 24


def DEBUG_GROUP_M(g: int) -> int:
    return (g & 0x3F) << 2


N_TILE_CONFIGS = 29
N_MX_CONFIGS = 8
MX_E4M3 = 0
MX_E2M1 = 1
N_SKINNY_CONFIGS = 6

VARIANT_NONE, VARIANT_TILE, VARIANT_SKINNY, VARIANT_MX = 0, 1, 2, 3


class Strides(ctypes.Structure):
    _fields_ = [("a_m", ctypes.c_int64), ("a_k", ctypes.c_int64),
                ("b_k", ctypes.c_int64), ("b_n", ctypes.c_int64),
                ("c_m", ctypes.c_int64), ("c_n", ctypes.c_int64)]


class Plan(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("config", ctypes.c_int32),
                ("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("bk", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("tiles_m", ctypes.c_int32), ("tiles_n", ctypes.c_int32),
                ("group_m", ctypes.c_int32), ("xcds", ctypes.c_int32),
                ("k_split", ctypes.c_int32), ("grid", ctypes.c_int64),
                ("tiles", ctypes.c_int64)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class TileGemmError(RuntimeError):
    def __init__(self, status, detail=""):
        self.status = Status(status)
        self.detail = detail
        super().__init__(f"{self.status.name}: {status_text(status)}"
                         + (f" ({detail})" if detail else ""))


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libtile_gemm.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise FileNotFoundError(
            f"{_LIB_PATH} is missing: build it with `python -m tile_partitioned_dense_amd.build`"
            " (there is no fallback implementation)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    P = ctypes.POINTER
    lib.tile_gemm_create.argtypes = [P(vp), i32]
    lib.tile_gemm_create.restype = i32
    lib.tile_gemm_destroy.argtypes = [vp]
    lib.tile_gemm_destroy.restype = i32
    lib.tile_gemm_run.argtypes = [vp, vp, vp, vp, i64, i64, i64, P(Strides), i32, vp]
    lib.tile_gemm_run.restype = i32
    lib.tile_gemm_run_debug.argtypes = [vp, vp, vp, vp, i64, i64, i64, P(Strides), i32, vp,
                                        vp, i32, vp, i32]
    lib.tile_gemm_run_debug.restype = i32
    lib.tile_gemm_run_epilogue.argtypes = [vp, vp, vp, vp, i64, i64, i64, P(Strides), i32, vp, i32,
                                           vp]
    lib.tile_gemm_run_epilogue.restype = i32
    lib.tile_gemm_check_epilogue.argtypes = [vp, i64, i64, P(Strides), i32, vp, i32]
    lib.tile_gemm_check_epilogue.restype = i32
    lib.tile_gemm_status_str.argtypes = [i32]
    lib.tile_gemm_status_str.restype = ctypes.c_char_p
    lib.tile_gemm_last_error_detail.argtypes = []
    lib.tile_gemm_last_error_detail.restype = ctypes.c_char_p
    lib.tile_gemm_check_args.argtypes = [vp, vp, vp, i64, i64, i64, P(Strides), i32]
    lib.tile_gemm_check_args.restype = i32
    lib.tile_gemm_plan.argtypes = [i64, i64, i64, i32, i32, P(Plan)]
    lib.tile_gemm_plan.restype = i32
    lib.tile_gemm_plan_mx.argtypes = [i64, i64, i64, i32, i32, P(Plan)]
    lib.tile_gemm_plan_mx.restype = i32
    lib.tile_gemm_run_mx.argtypes = [vp, vp, vp, vp, i64, i64, i64, P(Strides), vp, vp, i64, i32,
                                     i32, vp, i32, vp]
    lib.tile_gemm_run_mx.restype = i32
    lib.tile_gemm_run_mx_debug.argtypes = [vp, vp, vp, vp, i64, i64, i64, P(Strides), vp, vp, i64,
                                           i32, i32, vp, i32, vp, vp, i32]
    lib.tile_gemm_run_mx_debug.restype = i32
    lib.tile_gemm_check_mx.argtypes = [vp, vp, vp, i64, i64, i64, P(Strides), vp, vp, i64, i32, i32,
                                       vp, i32]
    lib.tile_gemm_check_mx.restype = i32
    lib.tile_gemm_tile_of.argtypes = [P(Plan), i64, i64, i64, P(i64), P(i64), P(i64), P(i64)]
    lib.tile_gemm_tile_of.restype = i32
    _lib = lib
    return lib


def status_text(s) -> str:
    return load_library().tile_gemm_status_str(int(s)).decode()


tile_gemm_status_str = status_text


def last_error_detail() -> str:
    return load_library().tile_gemm_last_error_detail().decode()


def _raise_if(st):
    if st != Status.OK:
        raise TileGemmError(st, last_error_detail())


# ----------------------------------------------------------------- handles

def tile_gemm_create(device: int = 0):
    """Create a handle for HIP device `device` (must be gfx950)."""
    lib = load_library()
    h = ctypes.c_void_p()
    _raise_if(lib.tile_gemm_create(ctypes.byref(h), int(device)))
    return h


def tile_gemm_destroy(h) -> None:
    _raise_if(load_library().tile_gemm_destroy(h))


# ----------------------------------------------------------------- marshalling

def _is_tensor(x):
    return hasattr(x, "data_ptr") and hasattr(x, "stride")


def _check_devices(named):
    """The library sees raw pointers only, so the binding checks what it cannot:
    every tensor argument lives on the GPU that is current (the device the
    library launches on), all on the same one. A host tensor's pointer handed
    to a kernel would fault the GPU."""
    import torch
    cur = torch.cuda.current_device() if torch.cuda.is_available() else None
    for name, t in named:
        if t is None or not _is_tensor(t):
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} is on {t.device}; every tensor argument must be on the GPU")
        if t.device.index != cur:
            raise ValueError(f"{name} is on {t.device}, but the current device is cuda:{cur}")


def _check_bias(bias, n):
    """A bias tensor must be a contiguous vector of n float32 values (the
    kernels read exactly that many)."""
    import torch
    if bias is None or not _is_tensor(bias):
        return
    if bias.dtype != torch.float32:
        raise TypeError(f"bias must be float32, got {bias.dtype}")
    if bias.dim() != 1 or bias.numel() != n or not bias.is_contiguous():
        raise ValueError(f"bias must be a contiguous vector of {n} values, got shape "
                         f"{tuple(bias.shape)} strides {tuple(bias.stride())}")


def _check_counts(counts, m, n):
    """Write counts: a contiguous 32-bit integer array of at least m*n elements."""
    import torch
    if counts is None or not _is_tensor(counts):
        return
    if counts.dtype not in (torch.int32, getattr(torch, "uint32", torch.int32)):
        raise TypeError(f"counts must be a 32-bit integer tensor, got {counts.dtype}")
    if counts.numel() < m * n or not counts.is_contiguous():
        raise ValueError(f"counts must be contiguous with at least {m * n} elements")


def _c_dtype(C):
    import torch
    if C.dtype == torch.float32:
        return Dtype.BF16_TO_F32
    if C.dtype == torch.bfloat16:
        return Dtype.BF16_TO_BF16
    raise TypeError("C must be float32 or bfloat16")


def _operands(A, B, C, M, N, K, strides, dtype, c_cols_div=1):
    """Pointers, shape, strides and dtype from torch tensors or raw values.
    C has N / c_cols_div columns (2 for SiLU(gate) * up)."""
    if _is_tensor(A) and _is_tensor(B) and _is_tensor(C):
        import torch
        if A.dim() != 2 or B.dim() != 2 or C.dim() != 2:
            raise ValueError("A, B and C must be 2-D")
        if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
            raise TypeError("A and B must be bfloat16")
        M_, K_ = A.shape
        K2, N_ = B.shape
        if K2 != K_ or N_ % c_cols_div or tuple(C.shape) != (M_, N_ // c_cols_div):
            raise ValueError(f"shapes do not chain: A{tuple(A.shape)} B{tuple(B.shape)} "
                             f"C{tuple(C.shape)}")
        cdt = _c_dtype(C)
        if dtype is None:
            dtype = cdt
        elif int(dtype) != cdt:
            raise TypeError(f"dtype {Dtype(int(dtype)).name} does not match C's {C.dtype}")
        s = Strides(A.stride(0), A.stride(1), B.stride(0), B.stride(1), C.stride(0), C.stride(1))
        return (A.data_ptr(), B.data_ptr(), C.data_ptr(), M_, N_, K_, s, int(dtype))
    if any(_is_tensor(x) for x in (A, B, C)):
        raise TypeError("A, B and C must be all torch tensors or all raw pointers")
    if None in (M, N, K, strides, dtype):
        raise ValueError("raw pointers need M, N, K, strides and dtype")
    s = strides if isinstance(strides, Strides) else Strides(*strides)
    return (A, B, C, int(M), int(N), int(K), s, int(dtype))


def _stream_ptr(stream, C):
    if stream is None:
        if _is_tensor(C) and C.is_cuda:
            import torch
            return torch.cuda.current_stream(C.device).cuda_stream
        return None
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


def tile_gemm_run(h, A, B, C, M=None, N=None, K=None, strides=None, dtype=None, stream=None,
                  check: bool = True):
    """Enqueue C := A.B. With torch tensors the shape, strides, output dtype and
    (unless given) the current stream are taken from them. Returns the status;
    raises TileGemmError on a non-OK status when `check` is true."""
    a, b, c, M_, N_, K_, s, dt = _operands(A, B, C, M, N, K, strides, dtype)
    _check_devices((("A", A), ("B", B), ("C", C)))
    st = load_library().tile_gemm_run(h, a, b, c, M_, N_, K_, ctypes.byref(s), dt,
                                      _stream_ptr(stream, C))
    if check:
        _raise_if(st)
    return Status(st)


def tile_gemm_run_epilogue(h, A, B, C, bias=None, act=Act.NONE, M=None, N=None, K=None,
                           strides=None, dtype=None, stream=None, check: bool = True):
    """Enqueue C := act(A.B + bias) (bias: N fp32 values on the device, or None).
    With act=Act.SWIGLU, C is M x N/2: silu of B's first N/2 columns' results
    times its last N/2."""
    div = 2 if int(act) == Act.SWIGLU else 1
    a, b, c, M_, N_, K_, s, dt = _operands(A, B, C, M, N, K, strides, dtype, div)
    _check_bias(bias, N_)
    _check_devices((("A", A), ("B", B), ("C", C), ("bias", bias)))
    bp = bias.data_ptr() if _is_tensor(bias) else bias
    st = load_library().tile_gemm_run_epilogue(h, a, b, c, M_, N_, K_, ctypes.byref(s), dt, bp,
                                               int(act), _stream_ptr(stream, C))
    if check:
        _raise_if(st)
    return Status(st)


def tile_gemm_run_debug(h, A, B, C, counts=None, flags=0, M=None, N=None, K=None, strides=None,
                        dtype=None, stream=None, check: bool = True, bias=None, act=Act.NONE):
    """tile_gemm_run (or, with bias/act, tile_gemm_run_epilogue) with test
    instrumentation (write counts, collision, forced configuration or grid)."""
    div = 2 if int(act) == Act.SWIGLU else 1
    a, b, c, M_, N_, K_, s, dt = _operands(A, B, C, M, N, K, strides, dtype, div)
    _check_bias(bias, N_)
    _check_counts(counts, M_, N_ // div)
    _check_devices((("A", A), ("B", B), ("C", C), ("bias", bias), ("counts", counts)))
    cnt = counts.data_ptr() if _is_tensor(counts) else counts
    bp = bias.data_ptr() if _is_tensor(bias) else bias
    st = load_library().tile_gemm_run_debug(h, a, b, c, M_, N_, K_, ctypes.byref(s), dt,
                                            _stream_ptr(stream, C), cnt, int(flags), bp,
                                            int(act))
    if check:
        _raise_if(st)
    return Status(st)


def _mx_operands(A, Bt, C, a_scale, b_scale, fmt=MX_E4M3):
    """Pointers, shape and strides of an MX call from torch tensors: A (M x K)
    and Bt (N x K) uint8 E4M3 codes (E2M1: M x K/2 and N x K/2 packed bytes),
    scales uint8 (M x ls) and (N x ls)."""
    import torch
    for name, t in (("A", A), ("Bt", Bt), ("a_scale", a_scale), ("b_scale", b_scale)):
        if t.dtype != torch.uint8 or t.dim() != 2:
            raise TypeError(f"{name} must be a 2-D uint8 tensor")
    M, K = A.shape
    N, K2 = Bt.shape
    if fmt == MX_E2M1:
        K, K2 = 2 * K, 2 * K2
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shapes do not chain: A{tuple(A.shape)} Bt{tuple(Bt.shape)} C{tuple(C.shape)}")
    if a_scale.shape[0] != M or b_scale.shape[0] != N or a_scale.stride(1) != 1 \
            or b_scale.stride(1) != 1:
        raise ValueError("scales: M and N rows with unit column stride")
    # One row stride serves both scale arrays. The stride of a single-row
    # array is never used (and torch may report any value for it), so it takes
    # the other array's; two single rows use their row length.
    if M > 1 and N > 1 and a_scale.stride(0) != b_scale.stride(0):
        raise ValueError("scales: A's and B's scale rows must have one common stride")
    ls = a_scale.stride(0) if M > 1 else (b_scale.stride(0) if N > 1 else a_scale.shape[1])
    dtype = _c_dtype(C)
    s = Strides(A.stride(0), A.stride(1), Bt.stride(1), Bt.stride(0), C.stride(0), C.stride(1))
    return M, N, K, s, ls, int(dtype)


def tile_gemm_run_mx(h, A, Bt, C, a_scale, b_scale, bias=None, act=Act.NONE, stream=None,
                     counts=None, flags=0, check: bool = True, fmt=MX_E4M3):
    """Enqueue the MX product C := act((sa * A) . (sb * Bt)^T + bias) (torch tensors)."""
    M, N, K, s, ls, dt = _mx_operands(A, Bt, C, a_scale, b_scale, fmt)
    _check_bias(bias, N)
    _check_counts(counts, M, N)
    _check_devices((("A", A), ("Bt", Bt), ("C", C), ("a_scale", a_scale), ("b_scale", b_scale),
                    ("bias", bias), ("counts", counts)))
    bp = bias.data_ptr() if _is_tensor(bias) else bias
    lib = load_library()
    args = (h, A.data_ptr(), Bt.data_ptr(), C.data_ptr(), M, N, K, ctypes.byref(s),
            a_scale.data_ptr(), b_scale.data_ptr(), ls, int(fmt), dt, bp, int(act),
            _stream_ptr(stream, C))
    if flags or counts is not None:
        cnt = counts.data_ptr() if _is_tensor(counts) else counts
        st = lib.tile_gemm_run_mx_debug(*args, cnt, int(flags))
    else:
        st = lib.tile_gemm_run_mx(*args)
    if check:
        _raise_if(st)
    return Status(st)


def tile_gemm_check_mx(A, B, C, M, N, K, strides, a_scale, b_scale, scale_stride, dtype,
                       bias=None, act=Act.NONE, fmt=MX_E4M3) -> Status:
    """Host-only checks of tile_gemm_run_mx's arguments (pointers are integers)."""
    s = strides if isinstance(strides, Strides) else Strides(*strides)
    return Status(load_library().tile_gemm_check_mx(A, B, C, int(M), int(N), int(K), ctypes.byref(s),
                                                    a_scale, b_scale, int(scale_stride), int(fmt),
                                                    int(dtype), bias, int(act)))


def tile_gemm_plan_mx(M, N, K, fmt=0, cu_count=256) -> Plan:
    p = Plan()
    _raise_if(load_library().tile_gemm_plan_mx(int(M), int(N), int(K), int(fmt), int(cu_count),
                                               ctypes.byref(p)))
    return p


def tile_gemm_check_args(A, B, C, M, N, K, strides, dtype) -> Status:
    """Host-only argument checks (pointers are plain integers here)."""
    s = strides if isinstance(strides, Strides) else Strides(*strides)
    return Status(load_library().tile_gemm_check_args(A, B, C, int(M), int(N), int(K),
                                                      ctypes.byref(s), int(dtype)))


def tile_gemm_check_epilogue(C, M, N, strides, dtype, bias, act) -> Status:
    """Host-only checks of the fused epilogue's arguments."""
    s = strides if isinstance(strides, Strides) else Strides(*strides)
    return Status(load_library().tile_gemm_check_epilogue(C, int(M), int(N), ctypes.byref(s),
                                                          int(dtype), bias, int(act)))


def tile_gemm_plan(M, N, K, b_col_major=False, cu_count=256) -> Plan:
    p = Plan()
    _raise_if(load_library().tile_gemm_plan(int(M), int(N), int(K), int(bool(b_col_major)),
                                            int(cu_count), ctypes.byref(p)))
    return p


def tile_gemm_tile_of(plan: Plan, M, N, wg):
    vals = [ctypes.c_int64() for _ in range(4)]
    _raise_if(load_library().tile_gemm_tile_of(ctypes.byref(plan), int(M), int(N), int(wg),
                                               *[ctypes.byref(v) for v in vals]))
    return tuple(v.value for v in vals)


class TileGemm:
    """Owns one handle; ``g(A, B, C)`` enqueues C := A.B on the current stream."""

    def __init__(self, device: int = 0):
        self.handle = tile_gemm_create(device)

    def __call__(self, A, B, C, stream=None, bias=None, act=None):
        if bias is None and act is None:
            return tile_gemm_run(self.handle, A, B, C, stream=stream)
        return tile_gemm_run_epilogue(self.handle, A, B, C, bias=bias,
                                      act=Act.NONE if act is None else act, stream=stream)

    def run_debug(self, A, B, C, counts=None, flags=0, stream=None, bias=None, act=None):
        return tile_gemm_run_debug(self.handle, A, B, C, counts=counts, flags=flags,
                                   stream=stream, bias=bias,
                                   act=Act.NONE if act is None else act)

    def mx(self, A, Bt, C, a_scale, b_scale, bias=None, act=None, stream=None, counts=None,
           flags=0, fmt=MX_E4M3):
        """MX product (tile_gemm_run_mx) into C."""
        return tile_gemm_run_mx(self.handle, A, Bt, C, a_scale, b_scale, bias=bias,
                                act=Act.NONE if act is None else act, stream=stream,
                                counts=counts, flags=flags, fmt=fmt)

    def close(self):
        if self.handle is not None:
            tile_gemm_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):  # pragma: no cover - best effort
        try:
            self.close()
        except Exception:
            pass
