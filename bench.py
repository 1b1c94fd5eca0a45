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
    ap.add_argument("--secondary", default="qkv_shard,square4096,decode,decode_colB,gemm256,"
                    "mx_mlp_gate_up_shard,mx_decode",
                    help="comma-separated extra workloads reported on the same line; NAME:EPI adds a "
                    "fused epilogue, e.g. decode:bias+silu ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time for the oracle baseline sample")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this size (for counter calibration)")
    return ap.parse_args()


class Bench:
    def __init__(self, torch, tg, synth):
        self.torch, self.tg, self.synth = torch, tg, synth
        self.g = tg.TileGemm(0)

    def make(self, w, out):
        torch, synth = self.torch, self.synth
        t0 = time.time()
        ops = synth.operands(w)
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
        for i in range(warmup):
            A, B, C = sets[i % len(sets)]
            g(A, B, C, **kw)
        torch.cuda.synchronize()
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            A, B, C = sets[i % len(sets)]
            starts[i].record()
            g(A, B, C, **kw)
            ends[i].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
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
        plan = self.tg.tile_gemm_plan(w.M, w.N, w.K, w.b_col_major, 256)
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
        if unfused is not None:
            res["unfused_torch_ms_mean"] = unfused
        mean_s = res["kernel_ms_mean"] * 1e-3
        res["tflops"] = w.flops / mean_s / 1e12
        res["gbs"] = w.algorithmic_bytes(out) / mean_s / 1e9
        res["frac_mfma"] = res["tflops"] / PEAK_BF16_TFLOPS
        res["frac_hbm"] = res["gbs"] / PEAK_HBM_GBS
        if w.flops < 1e9:
            res["launch_us"] = self.launch_overhead(sets[0])
        log(f"[bench] {w.name}: mean {res['kernel_ms_mean'] * 1e3:.1f} us "
            f"(median {res['kernel_ms_median'] * 1e3:.1f}, min {res['kernel_ms_min'] * 1e3:.1f}) "
            f"-> {res['tflops']:.1f} TFLOP/s ({100 * res['frac_mfma']:.1f}% MFMA), "
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
    for i in range(warmup):
        a, bt, sa, sb = sets[i % copies]
        g.mx(a, bt, Cs[i % copies], sa, sb, fmt=fmt)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        a, bt, sa, sb = sets[i % copies]
        ev[i][0].record()
        g.mx(a, bt, Cs[i % copies], sa, sb, fmt=fmt)
        ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([x.elapsed_time(y) for x, y in ev])
    plan = b.tg.tile_gemm_plan_mx(w.M, w.N, w.K, 256)
    res = {"workload": w.name, "M": w.M, "N": w.N, "K": w.K,
           "format": "MXFP4 (E2M1, E8M0 / 32)" if w.fmt == "e2m1" else "MXFP8 (E4M3, E8M0 / 32)",
           "out": out, "wall_ms_per_step": 1e3 * wall / steps,
           "kernel_ms_mean": float(per.mean()), "kernel_ms_median": float(np.median(per)),
           "kernel_ms_min": float(per.min()), "kernel_ms_max": float(per.max()),
           "flop": w.flops, "bytes": w.algorithmic_bytes(out),
           "plan": {"variant": "mx", "bm": plan.bm, "bn": plan.bn, "grid": int(plan.grid)}}
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
    head_out = head.outs[0]
    ops, res = b.time_workload(head, head_out, args.steps, args.warmup)
    secondary = []
    for name in [s for s in args.secondary.split(",") if s and s != args.workload]:
        if name in synth.MX_WORKLOADS:
            secondary.append(time_mx_workload(b, synth.MX_WORKLOADS[name], args.steps, args.warmup))
            continue
        base, _, epi = name.partition(":")
        w = synth.WORKLOADS[base]
        _, r = b.time_workload(w, w.outs[0], args.steps, args.warmup, epi or None)
        r["roofline"] = roofline(r, hbm_bound=name.startswith("decode"))
        secondary.append(r)
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
        "kernel_ms": {k: round(res[k], 5) for k in
                      ("kernel_ms_mean", "kernel_ms_median", "kernel_ms_min", "kernel_ms_max")},
        "secondary": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
                      for r in secondary],
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample of the headline workload")
        line["cpu_baseline"] = cpu_baseline(head, ops, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
