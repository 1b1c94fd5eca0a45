"""Build libtile_gemm.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Each kernel configuration is its own translation unit, compiled in parallel;
the objects are linked into ``tile_partitioned_dense_amd/libtile_gemm.so``.

    python -m tile_partitioned_dense_amd.build [--jobs N] [--save-temps]
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtile_gemm.so")
PROBES_LIB = os.path.join(PKG, "libtile_probes.so")   # measurement probes, not the GEMM ABI
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

N_TILE_CONFIGS = 29
N_SKINNY_CONFIGS = 6
N_MX_CONFIGS = 8

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


def _units():
    units = [("tile_gemm", os.path.join(CSRC, "tile_gemm.hip"), [])]
    for i in range(N_TILE_CONFIGS):
        units.append((f"kernels_tile_{i}", os.path.join(CSRC, "kernels_tile.hip"),
                      [f"-DTG_TILE_CONFIG={i}"]))
    for i in range(N_SKINNY_CONFIGS):
        units.append((f"kernels_skinny_{i}", os.path.join(CSRC, "kernels_skinny.hip"),
                      [f"-DTG_SKINNY_CONFIG={i}"]))
    for i in range(N_MX_CONFIGS):
        units.append((f"kernels_mx_{i}", os.path.join(CSRC, "kernels_mx.hip"),
                      [f"-DTG_MX_CONFIG={i}"]))
    return units


def _compile(unit, save_temps):
    name, src, defs = unit
    obj = os.path.join(BUILD, name + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *defs, "-c", src, "-o", obj]
    if save_temps:
        tdir = os.path.join(BUILD, "temps", name)
        os.makedirs(tdir, exist_ok=True)
        cmd += ["-save-temps=obj", f"-Rpass-analysis=kernel-resource-usage"]
        cmd[-1:-1] = []
        cmd = cmd[:-2] + ["-o", os.path.join(tdir, name + ".o")]
        r = subprocess.run(cmd, capture_output=True, text=True, cwd=tdir)
        shutil.copy(os.path.join(tdir, name + ".o"), obj)
    else:
        r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile {name} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stderr or "").splitlines() if noise not in ln]
    return obj, "\n".join(msgs)


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs: int | None = None, save_temps: bool = False, verbose: bool = False) -> str:
    """Compile every kernel unit and link the shared library. Always rebuilds."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(16, len(os.sched_getaffinity(0)))
    t0 = time.time()
    units = _units()
    objs = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, u, save_temps) for u in units]
        probe = ex.submit(_compile, ("probes", os.path.join(CSRC, "probes.hip"), []), False)
        for f in futs:
            obj, msg = f.result()
            objs.append(obj)
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
        probe_obj, _ = probe.result()
    _link([probe_obj], PROBES_LIB)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(objs)} units in {time.time() - t0:.1f}s", file=sys.stderr)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--save-temps", action="store_true",
                    help="keep the generated AMD assembly under _build/temps")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.save_temps, verbose=True))


if __name__ == "__main__":
    main()
