#!/usr/bin/env python3
"""Benchmark of the tile-partitioned GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one C = A.B over the headline workload's synthetic operands (the
planner, the owned-tile map, the LDS-staged K loop, MFMA and the owned-tile
store all run in it); the decode-shaped workload exercises the skinny
HBM-streaming kernel and is reported on the same line. Inputs are resident in
HBM before timing starts; each step uses the next of several copies of the
operands so that the 256 MB last-level cache cannot hold them between steps.

Prints ONE JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s & % MFMA peak (large); HBM GB/s & % peak (decode shape)"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_FP8_TFLOPS = 5033.2       # MI355X dense fp8 MFMA (twice the bf16 rate)
PEAK_FP4_TFLOPS = 10066.3      # MI355X dense fp4 / fp6 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
MIN_ROTATION_BYTES = 600 << 20  # > 2x the 256 MB last-level cache
CU_COUNT = 256                  # MI355X compute units
RIDGE_FLOP_PER_BYTE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # below: HBM-bound

# Secondary legs of the default run: the other bf16 workloads (4096^3 in both
# output types), the decode / tall-skinny sweep in both B layouts, the
# per-call cost on a ~1 us kernel, and the MX products in both formats.
DEFAULT_SECONDARY = ",".join([
    "qkv_shard", "square4096", "square4096@f32",
    "decode_m64", "decode_m32", "decode", "decode_m8", "decode_m1",
    "decode_colB_m64", "decode_colB_m32", "decode_colB", "decode_colB_m8", "decode_colB_m1",
    "tall_skinny", "tall_skinny_colB", "gemm256", "launch64",
    "mx_mlp_gate_up_shard", "mx_decode", "mxfp4_mlp_gate_up_shard", "mxfp4_decode",
])


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mlp_gate_up_shard")
    # Each default leg runs its own kernel instance, so a profiler's per-kernel
    # averages match the legs; epilogue legs (NAME:EPI, same instances as the
    # plain product) and mx_square4096 are available on request.
    ap.add_argument("--secondary", default=DEFAULT_SECONDARY,
                    help="comma-separated extra workloads reported on the same line; NAME:EPI adds a "
                    "fused epilogue, e.g. decode:bias+silu; NAME@f32 or NAME@bf16 picks the output "
                    "type ('' for none)")
    ap.add_argument("--k", type=int, default=0,
                    help="run the headline workload with this K instead (counter runs at two K "
                         "separate what a K step costs from what a tile's prologue and epilogue cost)")
    ap.add_argument("--probes", action="store_true",
                    help="also run the MFMA-rate and HBM streaming-read probes (libtile_probes.so)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time for the oracle baseline sample")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this size (for counter calibration)")
    return ap.parse_args()


class ClockProbe:
    """The average shader clock while a leg's timed launches run: a one-wave
    kernel (csrc/probes.hip, clock_probe) on a second stream reads the
    shader-cycle and real-time counters over a window that the timed launches
    cover. The real-time counter's rate is calibrated once against HIP events.
    Context for the roofline fractions: the published peaks assume 2.4 GHz."""

    def __init__(self, torch):
        import ctypes
        self.torch = torch
        self.lib = ctypes.CDLL(os.path.join(ROOT, "tile_partitioned_dense_amd", "libtile_probes.so"))
        self.lib.tg_probe_clock.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p]
        self.out = torch.zeros(2, dtype=torch.int64, device="cuda")
        self.side = torch.cuda.Stream()
        self.window_s = 0.0
        self.last = None
        # real-time ticks per second: a 2 ms-scale window timed with events
        ticks = 200000
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(2):
            e0.record()
            self._launch(ticks, torch.cuda.current_stream())
            e1.record()
            torch.cuda.synchronize()
        secs = e0.elapsed_time(e1) * 1e-3
        self.rt_hz = int(self.out[1].item()) / secs

    def _launch(self, ticks, stream):
        st = self.lib.tg_probe_clock(self.out.data_ptr(), int(ticks), stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"clock probe launch failed ({st})")

    def __call__(self, window_s, grid=0):
        """A window of about `window_s` seconds beside a kernel of `grid`
        workgroups. A kernel with a workgroup on every compute unit leaves no
        room for the probe's wave (each workgroup holds its unit's whole
        register file), so a probe would push one workgroup into a second
        round: then none is launched and the clock is not reported."""
        self.window_s = window_s
        self.active = grid < CU_COUNT
        return self

    def __enter__(self):
        torch = self.torch
        if not self.active:
            return self
        self.side.wait_stream(torch.cuda.current_stream())
        ticks = max(1000, min(int(self.window_s * self.rt_hz), 10 ** 9))
        self._launch(ticks, self.side)
        return self

    def __exit__(self, *exc):
        self.torch.cuda.synchronize()
        if not self.active:
            self.last = {"shader_clock_mhz": None,
                         "source": "not measured: the kernel's workgroups occupy every compute unit"}
            return
        cycles, ticks = (int(v) for v in self.out.tolist())
        self.last = {"shader_clock_mhz": round(cycles / (ticks / self.rt_hz) / 1e6, 1),
                     "window_ms": round(ticks / self.rt_hz * 1e3, 3),
                     "source": "s_memtime over s_memrealtime in a one-wave kernel beside the "
                               "timed launches"}

    def report(self):
        return self.last


class Bench:
    def __init__(self, torch, tg, synth):
        self.torch, self.tg, self.synth = torch, tg, synth
        self.g = tg.TileGemm(0)
        self.clock = ClockProbe(torch)
        self._host = {}

    def operands(self, w):
        """Host operands of a workload. The decode sweep's legs share the seeds
        of their layout, so B is the same draw and A's rows are the first rows
        of one stream: drawn once for the largest M (the default legs run that
        one first), sliced for the others."""
        key = (w.case, w.b_col_major, w.N, w.K)
        ops = self._host.get(key)
        if ops is None or ops.A.shape[0] < w.M:
            ops = self.synth.operands(w)
            self._host[key] = ops
        if ops.A.shape[0] != w.M:
            ops = self.synth.Operands(ops.A[:w.M], ops.B, ops.B_storage)
        return ops

    def make(self, w, out):
        torch, synth = self.torch, self.synth
        t0 = time.time()
        ops = self.operands(w)
        A = torch.from_numpy(ops.A.view(np.int16)).cuda().view(torch.bfloat16)
        Bs = torch.from_numpy(ops.B_storage.view(np.int16)).cuda().view(torch.bfloat16)
        odt = torch.float32 if out == "f32" else torch.bfloat16
        set_bytes = w.algorithmic_bytes(out)
        copies = max(1, min(8, -(-MIN_ROTATION_BYTES // set_bytes)))
        sets = []
        for i in range(copies):
            Ai = A if i == 0 else A.clone()
            Bi = Bs if i == 0 else Bs.clone()
            Bv = Bi.t() if w.b_col_major else Bi
            Ci = torch.empty((w.M, w.N), dtype=odt, device="cuda")
            sets.append((Ai, Bv, Ci))
        torch.cuda.synchronize()
        log(f"[bench] {w.name}: {w.M}x{w.N}x{w.K} out={out} copies={copies} "
            f"(operands ready in {time.time() - t0:.1f}s)")
        return ops, sets

    def launch_overhead(self, abc, n=400, per_graph=20):
        """Host-visible cost per call for a launch-bound shape: each call
        followed by a synchronisation; calls chained on the stream with one
        synchronisation at the end; and the same calls captured into a HIP
        graph (per_graph per graph) and replayed."""
        torch, g = self.torch, self.g
        A, B, C = abc
        for _ in range(10):
            g(A, B, C)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            g(A, B, C)
            torch.cuda.synchronize()
        synced = (time.perf_counter() - t0) / n
        t0 = time.perf_counter()
        for _ in range(n):
            g(A, B, C)
        torch.cuda.synchronize()
        chained = (time.perf_counter() - t0) / n
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            g(A, B, C)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(per_graph):
                g(A, B, C)
        graph.replay()
        torch.cuda.synchronize()
        reps = max(1, n // per_graph)
        t0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        replay = (time.perf_counter() - t0) / (reps * per_graph)
        out = {"synced": round(synced * 1e6, 2), "chained": round(chained * 1e6, 2),
               "graph_replay": round(replay * 1e6, 2)}
        log(f"[bench] per-call cost (us): {out}")
        return out

    def time_workload(self, w, out, steps, warmup, epi=None):
        """Time `steps` launches of the product over rotating operand sets. `epi`
        names a fused epilogue ("bias+silu", "relu", ...): the timed call is
        then tile_gemm_run_epilogue, and the same product followed by torch's
        separate bias-add and activation pass is timed beside it."""
        torch = self.torch
        ops, sets = self.make(w, out)
        g = self.g
        kw = {}
        if epi:
            parts = epi.split("+")
            acts = [p for p in parts if p != "bias"]
            act = self.tg.Act[acts[0].upper()] if acts else self.tg.Act.NONE
            bias = (torch.from_numpy(self.synth.draw_bias(w.N, 760)).cuda()
                    if "bias" in parts else None)
            kw = {"bias": bias, "act": act}
            if act == self.tg.Act.SWIGLU:
                # the output is M x N/2; keep the full-width C for the unfused leg
                sets = [(A, B, torch.empty((w.M, w.N // 2), dtype=C.dtype, device="cuda"), C)
                        for A, B, C in sets]
        full_c = {i: (s[3] if len(s) > 3 else s[2]) for i, s in enumerate(sets)}
        sets = [s[:3] for s in sets]
        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0.record()
        for i in range(warmup):
            A, B, C = sets[i % len(sets)]
            g(A, B, C, **kw)
        w1.record()
        torch.cuda.synchronize()
        est = w0.elapsed_time(w1) * 1e-3 / max(warmup, 1)
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        torch.cuda.synchronize()
        plan = self.tg.tile_gemm_plan(w.M, w.N, w.K, w.b_col_major, CU_COUNT)
        with self.clock(0.7 * est * steps, plan.grid):
            t0 = time.perf_counter()
            for i in range(steps):
                A, B, C = sets[i % len(sets)]
                starts[i].record()
                g(A, B, C, **kw)
                ends[i].record()
            torch.cuda.current_stream().synchronize()   # the launching stream, not the probe's
            wall = time.perf_counter() - t0
        clock = self.clock.report()
        per = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])  # ms per launch
        unfused = None
        if epi:
            silu = torch.nn.functional.silu
            fn = {"none": lambda x: x, "relu": torch.relu, "sigmoid": torch.sigmoid,
                  "tanh": torch.tanh, "silu": silu,
                  "swiglu": lambda x: silu(x[:, :w.N // 2]) * x[:, w.N // 2:]}[
                      kw["act"].name.lower()]
            t = []
            for i in range(steps + warmup):
                A, B, _ = sets[i % len(sets)]
                C = full_c[i % len(sets)]
                s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s0.record()
                g(A, B, C)
                y = fn(C + kw["bias"]) if kw["bias"] is not None else fn(C)
                s1.record()
                t.append((s0, s1))
            torch.cuda.synchronize()
            unfused = float(np.mean([a.elapsed_time(b) for a, b in t[warmup:]]))
            del y
        res = {
            "workload": w.name + (f":{epi}" if epi else ""), "M": w.M, "N": w.N, "K": w.K,
            "b_layout": "column-major" if w.b_col_major else "row-major", "out": out,
            "wall_ms_per_step": 1e3 * wall / steps,
            "kernel_ms_mean": float(per.mean()), "kernel_ms_median": float(np.median(per)),
            "kernel_ms_min": float(per.min()), "kernel_ms_max": float(per.max()),
            "flop": w.flops, "bytes": w.algorithmic_bytes(out),
            "plan": {"variant": "tile" if plan.variant == 1 else "skinny", "bm": plan.bm,
                     "bn": plan.bn, "grid": int(plan.grid), "k_split": plan.k_split},
        }
        res["clock"] = clock
        if unfused is not None:
            res["unfused_torch_ms_mean"] = unfused
        mean_s = res["kernel_ms_mean"] * 1e-3
        res["tflops"] = w.flops / mean_s / 1e12
        res["gbs"] = w.algorithmic_bytes(out) / mean_s / 1e9
        res["frac_mfma"] = res["tflops"] / PEAK_BF16_TFLOPS
        res["frac_hbm"] = res["gbs"] / PEAK_HBM_GBS
        if w.flops < 1e8:
            res["launch_us"] = self.launch_overhead(sets[0])
        mhz = clock.get("shader_clock_mhz")
        log(f"[bench] {w.name}: mean {res['kernel_ms_mean'] * 1e3:.1f} us "
            f"(median {res['kernel_ms_median'] * 1e3:.1f}, min {res['kernel_ms_min'] * 1e3:.1f}) "
            + (f"at {mhz:.0f} MHz " if mhz else "(clock not sampled: the grid fills every CU) ")
            + f"-> {res['tflops']:.1f} TFLOP/s ({100 * res['frac_mfma']:.1f}% MFMA), "
            f"{res['gbs']:.0f} GB/s ({100 * res['frac_hbm']:.1f}% HBM)")
        del sets
        torch.cuda.empty_cache()
        return ops, res


def time_mx_workload(b, w, steps, warmup):
    """Time the MXFP8 product on an MX workload (operands rotated like the
    bf16 ones; elements, scales and C resident in HBM)."""
    torch, synth, g = b.torch, b.synth, b.g
    t0 = time.time()
    ops = synth.mx_operands(w)
    A = torch.from_numpy(ops.A).cuda()
    Bt = torch.from_numpy(ops.Bt).cuda()
    sA = torch.from_numpy(ops.sA).cuda()
    sB = torch.from_numpy(ops.sB).cuda()
    out = w.outs[0]
    odt = torch.float32 if out == "f32" else torch.bfloat16
    copies = max(1, min(8, -(-MIN_ROTATION_BYTES // w.algorithmic_bytes(out))))
    sets = [(A, Bt, sA, sB) if i == 0 else (A.clone(), Bt.clone(), sA.clone(), sB.clone())
            for i in range(copies)]
    Cs = [torch.empty((w.M, w.N), dtype=odt, device="cuda") for _ in range(copies)]
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: {w.M}x{w.N}x{w.K} {w.fmt} out={out} copies={copies} "
        f"(operands ready in {time.time() - t0:.1f}s)")
    fmt = b.tg.MX_E2M1 if w.fmt == "e2m1" else b.tg.MX_E4M3
    peak = PEAK_FP4_TFLOPS if w.fmt == "e2m1" else PEAK_FP8_TFLOPS
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record()
    for i in range(warmup):
        a, bt, sa, sb = sets[i % copies]
        g.mx(a, bt, Cs[i % copies], sa, sb, fmt=fmt)
    w1.record()
    torch.cuda.synchronize()
    est = w0.elapsed_time(w1) * 1e-3 / max(warmup, 1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    plan = b.tg.tile_gemm_plan_mx(w.M, w.N, w.K, fmt, CU_COUNT)
    with b.clock(0.7 * est * steps, plan.grid):
        t0 = time.perf_counter()
        for i in range(steps):
            a, bt, sa, sb = sets[i % copies]
            ev[i][0].record()
            g.mx(a, bt, Cs[i % copies], sa, sb, fmt=fmt)
            ev[i][1].record()
        torch.cuda.current_stream().synchronize()
        wall = time.perf_counter() - t0
    per = np.array([x.elapsed_time(y) for x, y in ev])
    res = {"workload": w.name, "M": w.M, "N": w.N, "K": w.K,
           "format": "MXFP4 (E2M1, E8M0 / 32)" if w.fmt == "e2m1" else "MXFP8 (E4M3, E8M0 / 32)",
           "out": out, "wall_ms_per_step": 1e3 * wall / steps,
           "kernel_ms_mean": float(per.mean()), "kernel_ms_median": float(np.median(per)),
           "kernel_ms_min": float(per.min()), "kernel_ms_max": float(per.max()),
           "flop": w.flops, "bytes": w.algorithmic_bytes(out),
           "plan": {"variant": "mx", "bm": plan.bm, "bn": plan.bn, "grid": int(plan.grid)},
           "clock": b.clock.report()}
    mean_s = res["kernel_ms_mean"] * 1e-3
    res["tflops"] = w.flops / mean_s / 1e12
    res["gbs"] = w.algorithmic_bytes(out) / mean_s / 1e9
    hbm = w.name.endswith("decode")
    res["roofline"] = ({"bound": "hbm", "achieved": round(res["gbs"], 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(res["gbs"] / PEAK_HBM_GBS, 4),
                        "traffic": measured_traffic(w.name)} if hbm else
                       {"bound": "mfma", "achieved": round(res["tflops"], 1),
                        "peak": peak, "unit": "TFLOP/s",
                        "frac": round(res["tflops"] / peak, 4),
                        "traffic": measured_traffic(w.name)})
    log(f"[bench] {w.name}: mean {res['kernel_ms_mean'] * 1e3:.1f} us -> {res['tflops']:.1f} "
        f"TFLOP/s ({100 * res['tflops'] / peak:.1f}% of {w.fmt} MFMA), {res['gbs']:.0f} GB/s")
    del sets, Cs
    torch.cuda.empty_cache()
    return res


def measured_traffic(workload):
    """HBM-side bytes per launch recorded by rocprofv3 counter runs
    (profiles/traffic.json), or None when the kernel sources have changed
    since those counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
        h = hashlib.sha256()
        for src in rec["kernel_sources"]:
            h.update(open(os.path.join(ROOT, src), "rb").read())
        if h.hexdigest() != rec["kernel_source_sha256"]:
            return None
        w = rec["workloads"][workload]
        return int(round(1024 * (w["fetch_kib"] * rec["fetch_scale"] + w["write_kib"] * rec["write_scale"])))
    except (OSError, KeyError, ValueError):
        return None


def run_probes(torch, clock):
    """The MFMA-rate, LDS-read and HBM streaming-read probes
    (csrc/probes.hip): the ceilings the GEMM kernels meet on this machine, beside
    the published peaks."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "tile_partitioned_dense_amd", "libtile_probes.so"))
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.tg_probe_mfma.argtypes = [vp, vp, i32, i32, i32, i32, vp]
    lib.tg_probe_read.argtypes = [vp, vp, i64, i32, i32, vp]
    lib.tg_probe_lds.argtypes = [vp, i32, i32, i32, vp]
    stream = torch.cuda.current_stream().cuda_stream
    grid = 256
    out = torch.empty(grid * 512, dtype=torch.float32, device="cuda")
    # 16 KiB of operands per wave (two waves per SIMD): bf16 N(0,1) values,
    # read by the E4M3 shapes as bytes (random codes) or, for constant
    # operands, bf16 1.0 = bytes 0x80 0x3f (E4M3 -0 and 1.875)
    rnd = torch.randn(grid * 8 * 16 * 1024 // 2, device="cuda").to(torch.bfloat16)
    const = torch.full_like(rnd, 1.0)

    def timed(fn, n=20, warm=3, grid_of_fn=0):
        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0.record()
        for _ in range(warm):
            fn()
        w1.record()
        torch.cuda.synchronize()
        est = w0.elapsed_time(w1) * 1e-3 / warm
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        with clock(0.7 * est * n, grid_of_fn):
            for a, b in ev:
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3, clock.report()

    mfma = []
    for shape, sname in ((0, "v_mfma_f32_32x32x16_bf16"), (1, "v_mfma_f32_16x16x32_bf16"),
                         (2, "v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3)"),
                         (3, "v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3)"),
                         (4, "v_mfma_scale_f32_32x32x64_f8f6f4 (E2M1)"),
                         (5, "v_mfma_scale_f32_16x16x128_f8f6f4 (E2M1)")):
        f8 = shape >= 2
        peak = PEAK_FP4_TFLOPS if shape >= 4 else PEAK_FP8_TFLOPS if f8 else PEAK_BF16_TFLOPS
        for wps in (1, 2):
            for data, src in (("random N(0,1)", rnd), ("constant 1.0", const)):
                iters = (1200 if f8 else 2400) // wps
                fn = lambda: lib.tg_probe_mfma(src.data_ptr(), out.data_ptr(), grid, wps, shape,
                                               iters, stream)
                t, clk = timed(fn)
                flop = grid * 4 * wps * iters * 64 * 32768 * (4 if f8 else 1)
                tf = flop / t / 1e12
                mhz = clk["shader_clock_mhz"]
                mfma.append({"instruction": sname, "waves_per_simd": wps, "operands": data,
                             "launch_ms": round(t * 1e3, 3), "tflops": round(tf, 1),
                             "frac_of_peak": round(tf / peak, 4),
                             "shader_clock_mhz": mhz,
                             "mfma_busy_at_that_clock": round(tf / (peak * mhz / 2400.0), 4)})
                log(f"[probe] {sname} {wps} wave(s)/SIMD {data}: {tf:.0f} TFLOP/s at {mhz:.0f} MHz")
    del rnd, const
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(7)
    rout = torch.empty(8192 * 256, dtype=torch.int32, device="cuda")
    read = []
    for chunk, g in ((1, 256), (1, 512), (1, 1024), (1, 2048), (0, 2048), (0, 8192)):
        fn = lambda: lib.tg_probe_read(buf.data_ptr(), rout.data_ptr(), nbytes, g, chunk, stream)
        t, clk = timed(fn, n=10)
        gbs = nbytes / t / 1e9
        read.append({"pattern": "one contiguous chunk per workgroup" if chunk else "grid-strided",
                     "workgroups": g, "bytes": nbytes, "launch_ms": round(t * 1e3, 3),
                     "gbs": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
                     "shader_clock_mhz": clk["shader_clock_mhz"]})
        log(f"[probe] read {read[-1]['pattern']} x{g}: {gbs:.0f} GB/s")
    del buf
    torch.cuda.empty_cache()
    lout = torch.empty(grid * 1024, dtype=torch.int32, device="cuda")
    lds = []
    for iters in (4096, 16384):
        fn = lambda: lib.tg_probe_lds(lout.data_ptr(), grid, iters, 1024, stream)
        t, clk = timed(fn, n=10)
        nbytes = grid * 16 * iters * 8 * 1024
        mhz = clk["shader_clock_mhz"]
        per_cu_clk = nbytes / grid / (t * mhz * 1e6) if mhz else None
        lds.append({"reads_per_wave": iters * 8, "bytes": nbytes, "launch_ms": round(t * 1e3, 3),
                    "gbs": round(nbytes / t / 1e9, 1), "shader_clock_mhz": mhz,
                    "bytes_per_cu_per_clock": round(per_cu_clk, 1) if per_cu_clk else None})
        log(f"[probe] lds read x{iters * 8}/wave: {nbytes / t / 1e9:.0f} GB/s, "
            f"{per_cu_clk if per_cu_clk else float('nan'):.1f} B per CU per clock at {mhz:.0f} MHz")
    return {"mfma": mfma, "hbm_read": read, "lds_read": lds}


def roofline(res, hbm_bound):
    traffic = measured_traffic(res["workload"])
    if hbm_bound:
        return {"bound": "hbm", "achieved": round(res["gbs"], 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(res["frac_hbm"], 4), "traffic": traffic}
    return {"bound": "mfma", "achieved": round(res["tflops"], 1), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(res["frac_mfma"], 4), "traffic": traffic}


def cpu_baseline(w, ops, seconds):
    """The fp64 triple-loop oracle, as it stands, on the first rows of the same
    operands; rows chosen for roughly `seconds` of CPU time."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    oracle.build(force=False)
    def run(rows):
        t0 = time.perf_counter()
        oracle.gemm(ops.A[:rows], ops.B, want_d=False, threads=threads)
        return time.perf_counter() - t0

    # rows run in parallel, one per thread: two probes of one and three rows
    # per thread give the cost of a round of rows and the fixed cost (the
    # decode of B); then time whole rounds for about `seconds`
    t1, t3 = run(threads), run(3 * threads)
    per_round = max((t3 - t1) / 2, 1e-6)
    fixed = max(t1 - per_round, 0.0)
    rounds = int(max(1, (seconds - fixed) / per_round))
    rows = int(min(w.M, rounds * threads))
    t = run(rows)
    flop = 2.0 * rows * w.N * w.K
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(flop / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"first {rows} of {w.M} rows of {w.name} ({w.M}x{w.N}x{w.K}), fp64 triple "
                      f"loop incl. its B decode, C only, {t:.2f}s wall on {cpu} "
                      f"({platform.machine()})",
            "seconds": round(t, 3)}


def copy_calibration(torch, mib):
    """A plain device copy of `mib` MiB, for scaling the HBM byte counters.
    A 512 MiB scratch write between the fill and the copy pushes the source
    out of the last-level cache, so the copy reads it from HBM."""
    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    flush = torch.empty(128 << 20, dtype=torch.float32, device="cuda")
    flush.fill_(2.0)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del flush
    log(f"[bench] copy calibration: {mib} MiB read + {mib} MiB written")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this library has no "
              "multi-GPU path", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    import tile_partitioned_dense_amd as tg
    from tile_partitioned_dense_amd import synth
    tg.load_library()

    b = Bench(torch, tg, synth)
    head = synth.WORKLOADS[args.workload]
    if args.k:
        import dataclasses
        head = dataclasses.replace(head, name=f"{head.name}@K{args.k}", K=args.k)
    head_out = head.outs[0]
    ops, res = b.time_workload(head, head_out, args.steps, args.warmup)
    secondary = []
    for name in [s for s in args.secondary.split(",") if s and s != args.workload]:
        if name in synth.MX_WORKLOADS:
            secondary.append(time_mx_workload(b, synth.MX_WORKLOADS[name], args.steps, args.warmup))
            continue
        base, _, epi = name.partition(":")
        base, _, out = base.partition("@")
        w = synth.WORKLOADS[base]
        _, r = b.time_workload(w, out or w.outs[0], args.steps, args.warmup, epi or None)
        if out:
            r["workload"] = f"{base}@{out}" + (f":{epi}" if epi else "")
        r["roofline"] = roofline(r, hbm_bound=w.flops / r["bytes"] < RIDGE_FLOP_PER_BYTE)
        secondary.append(r)
    probes = run_probes(torch, b.clock) if args.probes else None
    if args.copy_calibration_mib:
        copy_calibration(torch, args.copy_calibration_mib)

    hbm_head = head.name.startswith("decode")
    line = {
        "metric": METRIC,
        "value": round(res["gbs"] if hbm_head else res["tflops"], 2),
        "unit": "GB/s" if hbm_head else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["wall_ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head.name, "M": head.M, "N": head.N, "K": head.K,
                   "b_layout": res["b_layout"], "out": head_out, "parallelism": "none (1 GPU)",
                   "plan": res["plan"]},
        "roofline": roofline(res, hbm_head),
        "clock": res["clock"],
        "kernel_ms": {k: round(res[k], 5) for k in
                      ("kernel_ms_mean", "kernel_ms_median", "kernel_ms_min", "kernel_ms_max")},
        "secondary": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
                      for r in secondary],
    }
    if probes is not None:
        line["probes"] = probes
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample of the headline workload")
        line["cpu_baseline"] = cpu_baseline(head, ops, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
