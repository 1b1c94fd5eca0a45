"""Measure every tile configuration's rate on one shape: the numbers behind
the `eff` column of the planner's table (`kTileConfigs` in csrc/plan.hpp).

    python -m tile_partitioned_dense_amd.rate_configs [--shape 8192x7168x8192]
        [--bcol] [--out bf16|f32] [--rounds 5] [--launches 6] [--configs 7,17,19]

Each configuration that applies to the shape (the stream configurations need
a column-major B and an even K) is run with the library's debug entry forcing
it (the production kernel instances, only the choice of configuration is
overridden), in rotation with the others launch by launch so that drifts of
the shader clock and of the box hit every configuration alike, on rotating
copies of seeded random bf16 operands resident in HBM. A configuration's rate
is what the planner's cost model divides by: (tiles on the busiest compute
unit) x BM x BN / mean launch time, printed relative to configuration 7, the
table's unit. The planner applies the rate of a workgroup alone on its unit
(`eff1`) when there is one tile per unit and `eff` otherwise, so the shape
chosen decides which of the two a run measures.

Needs a GPU; the library is the one built in the package directory.
"""

import argparse
import os
import re
import sys

import numpy as np

CU_COUNT = 256
HERE = os.path.dirname(os.path.abspath(__file__))


def config_table():
    """(bm, bn, wm, wn, stages, eff, ks, eff1, occ, sb, mi, bk) for every entry
    of kTileConfigs, read from csrc/plan.hpp with the struct's defaults."""
    src = open(os.path.join(HERE, "csrc", "plan.hpp")).read()
    body = re.search(r"kTileConfigs\[kNumTileConfigs\]\s*=\s*\{(.*?)\n\};", src, re.S).group(1)
    rows = []
    for r in re.findall(r"^\s*\{([^}]*)\}", body, re.M):
        f = [x.strip().rstrip("f") for x in r.split(",")]
        defaults = ["1", "0.0", "1", "0", "32", "32"]  # ks, eff1, occ, sb, mi, bk
        f = f + defaults[len(f) - 6:]
        rows.append(dict(bm=int(f[0]), bn=int(f[1]), wm=int(f[2]), wn=int(f[3]), stages=int(f[4]),
                         eff=float(f[5]), ks=int(f[6]), eff1=float(f[7]), occ=int(f[8]), sb=int(f[9]),
                         mi=int(f[10]), bk=int(f[11])))
    return rows


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--shape", default="8192x7168x8192")
    ap.add_argument("--bcol", action="store_true", help="column-major B (default row-major)")
    ap.add_argument("--out", choices=("bf16", "f32"), default="bf16")
    ap.add_argument("--rounds", type=int, default=5)
    ap.add_argument("--launches", type=int, default=6, help="launches per configuration and round")
    ap.add_argument("--configs", default="", help="comma-separated indices (default: all that apply)")
    ap.add_argument("--seed", type=int, default=1234)
    args = ap.parse_args(argv)

    import torch
    sys.path.insert(0, os.path.dirname(HERE))
    import tile_partitioned_dense_amd as tg

    if not torch.cuda.is_available():
        print("rate_configs needs a GPU", file=sys.stderr)
        return 1
    M, N, K = (int(v) for v in args.shape.lower().split("x"))
    table = config_table()
    assert len(table) == tg.N_TILE_CONFIGS, "plan.hpp table and library disagree"
    if args.configs:
        cfgs = [int(c) for c in args.configs.split(",")]
    else:
        cfgs = [i for i, c in enumerate(table) if not c["sb"] or (args.bcol and K % 2 == 0)]
    if 7 not in cfgs:
        cfgs = [7] + cfgs

    gen = torch.Generator(device="cuda").manual_seed(args.seed)
    odt = torch.bfloat16 if args.out == "bf16" else torch.float32
    sets = []
    for _ in range(3):  # > 3 x the last-level cache for the large shapes
        A = torch.randn(M, K, generator=gen, device="cuda").to(torch.bfloat16)
        Bs = (torch.randn(N, K, generator=gen, device="cuda") / np.sqrt(K)).to(torch.bfloat16)
        B = Bs.t() if args.bcol else Bs.t().contiguous()
        sets.append((A, B, torch.empty(M, N, dtype=odt, device="cuda")))
    g = tg.TileGemm(0)
    times = {c: [] for c in cfgs}
    for c in cfgs:  # warm-up (and a first check that each configuration runs)
        g.run_debug(*sets[0], flags=tg.DEBUG_FORCE_TILE(c))
    torch.cuda.synchronize()
    n = 0
    for _ in range(args.rounds):
        for c in cfgs:
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.launches)]
            for e0, e1 in ev:
                A, B, C = sets[n % len(sets)]
                n += 1
                e0.record()
                g.run_debug(A, B, C, flags=tg.DEBUG_FORCE_TILE(c))
                e1.record()
            torch.cuda.synchronize()
            times[c] += [e0.elapsed_time(e1) * 1e-3 for e0, e1 in ev]

    def rate(c, t):
        cfg = table[c]
        tiles = -(-M // cfg["bm"]) * -(-N // cfg["bn"])
        per_cu = -(-tiles // CU_COUNT)
        return per_cu * cfg["bm"] * cfg["bn"] / t, per_cu

    ref, _ = rate(7, float(np.mean(times[7])))
    print(f"# rates on {M}x{N}x{K}, B {'column' if args.bcol else 'row'}-major, {args.out} out, "
          f"{args.rounds} rounds x {args.launches} launches per configuration")
    print("| config | tile | waves | MFMA | K slab | mean us | min us | TFLOP/s | tiles per CU "
          "| rate / config 7 | table eff (eff1) |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for c in cfgs:
        cfg = table[c]
        t = float(np.mean(times[c]))
        r, per_cu = rate(c, t)
        waves = cfg["wm"] * cfg["wn"] * cfg["ks"]
        mfma = "16x16x32" if cfg["mi"] == 16 else "32x32x16"
        slab = cfg["sb"] // 2 if cfg["sb"] else cfg["bk"]
        e1 = f" ({cfg['eff1']:.2f})" if cfg["eff1"] else ""
        print(f"| {c} | {cfg['bm']}x{cfg['bn']} | {waves} | {mfma} | {slab} | {t * 1e6:.1f} | "
              f"{min(times[c]) * 1e6:.1f} | {2 * M * N * K / t / 1e12:.0f} | {per_cu} | {r / ref:.3f} | "
              f"{cfg['eff']:.2f}{e1} |")
    return 0


if __name__ == "__main__":
    sys.exit(main())
