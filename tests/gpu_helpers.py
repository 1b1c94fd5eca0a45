"""Helpers shared by the GPU tests: seeded operands on the device, padded
layouts, and the oracle's expected values (computed on the CPU from the same
bits). Nothing here computes the product."""

from __future__ import annotations

import numpy as np

import oracle
from tile_partitioned_dense_amd import synth


def torch_mod():
    import torch
    return torch


def dev_bf16(bits: np.ndarray, device="cuda:0"):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)
    return t.view(torch.bfloat16)


def host_bits(t) -> np.ndarray:
    torch = torch_mod()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host_out(C) -> np.ndarray:
    torch = torch_mod()
    if C.dtype == torch.float32:
        return C.cpu().numpy()
    return host_bits(C)


def tile_config_table():
    """(bm, bn, wm, wn, stages) of every compiled tile configuration, read from
    the planner's table so new configurations are covered automatically."""
    import os
    import re
    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "tile_partitioned_dense_amd", "csrc", "plan.hpp")).read()
    body = re.search(r"kTileConfigs\[kNumTileConfigs\]\s*=\s*\{(.*?)\n\};", src, re.S).group(1)
    rows = re.findall(r"^\s*\{(\d+),\s*(\d+),\s*(\d+),\s*(\d+),\s*(\d+),", body, re.M)
    return [tuple(int(v) for v in r) for r in rows]


def stream_tile_configs():
    """Indices of the tile configurations that run the stream kernel (a field
    sb > 0, the tenth of a row): column-major B only."""
    import os
    import re
    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "tile_partitioned_dense_amd", "csrc", "plan.hpp")).read()
    body = re.search(r"kTileConfigs\[kNumTileConfigs\]\s*=\s*\{(.*?)\n\};", src, re.S).group(1)
    rows = [[f.strip() for f in r.split(",")] for r in re.findall(r"^\s*\{([^}]*)\}", body, re.M)]
    return {i for i, r in enumerate(rows) if len(r) > 9 and int(r[9]) > 0}


def round_up(x, m):
    return (x + m - 1) // m * m


class Case:
    """Seeded operands for one shape with padded leading dimensions, held both
    as numpy bit views (for the oracle) and as device views (for the GPU)."""

    def __init__(self, M, N, K, b_col_major=False, dist="normal", seed=0, pad=0,
                 b_scale=1.0, device="cuda:0"):
        self.M, self.N, self.K, self.bcol = M, N, K, b_col_major
        lda = round_up(max(K, 1), 8) + pad
        A_store = synth.draw(M, lda, dist, 2 * seed + 1)
        self.A = A_store[:, :K]
        if b_col_major:
            ldb = round_up(max(K, 1), 8) + pad
            B_store = synth.draw(N, ldb, dist, 2 * seed + 2, b_scale)
            self.B = B_store[:, :K].T
        else:
            ldb = round_up(max(N, 1), 8) + pad
            B_store = synth.draw(K, ldb, dist, 2 * seed + 2, b_scale)
            self.B = B_store[:, :N]
        self.A_dev = dev_bf16(A_store, device)[:, :K]
        Bd = dev_bf16(B_store, device)
        self.B_dev = Bd[:, :K].t() if b_col_major else Bd[:, :N]
        self.pad = pad
        self.device = device
        self._ref = None

    def out(self, dtype, fill=float("nan")):
        """A padded output view (padding columns hold the sentinel too)."""
        torch = torch_mod()
        ld = round_up(max(self.N, 1), 8) + self.pad
        store = torch.full((self.M, ld), fill, dtype=dtype, device=self.device)
        return store, store[:, : self.N]

    def ref(self, blas=False):
        if self._ref is None:
            self._ref = oracle.gemm_blas(self.A, self.B) if blas else oracle.gemm(self.A, self.B)
        return self._ref


def workload_case(name, integer=False, device="cuda:0"):
    """Operands of a named workload at full size (numpy views + device views)."""
    w = synth.WORKLOADS[name]
    ops = synth.operands(w, integer=integer)
    A_dev = dev_bf16(ops.A, device)
    Bs = dev_bf16(ops.B_storage, device)
    B_dev = Bs.t() if w.b_col_major else Bs
    return w, ops, A_dev, B_dev


def check(out_np, C, D, bf16, integer=False, rel=1e-5):
    if integer:
        return oracle.check_exact(out_np, C, bf16)
    return oracle.check_bf16(out_np, C, D, rel) if bf16 else oracle.check_f32(out_np, C, D, rel)
