"""Build libmiattn.so for gfx950 with hipcc (in-tree, next to this file).

Each csrc/*.hip file is compiled to an object in parallel, then all objects
are linked into exact_tiled_attention_09_amd/libmiattn.so.  Usage:

    python -m exact_tiled_attention_09_amd.build [--jobs N] [--verbose]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmiattn.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-variable",
    # packed fp32 VALU forms are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
    f"-I{CSRC}",
]


# Extra flags per source.  The backward kernel keeps its dK/dV accumulators
# live across the query-tile loop; in AGPR form the compiler copies them
# between register files every iteration, the VGPR form does not.
FILE_FLAGS = {
    "bwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libmiattn)")
    return path


def _compile(src: str, obj: str, verbose: bool) -> tuple[str, float]:
    t0 = time.time()
    cmd = [hipcc(), *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{res.stdout}\n{res.stderr}")
    noise = "is not a recognized feature for this target"
    warn = "\n".join(line for line in res.stderr.splitlines() if line.strip() and noise not in line)
    if warn and verbose:
        print(warn, file=sys.stderr)
    return src, time.time() - t0


PROBE_SRC = os.path.join(PKG, "calib", "mfma_probe.hip")
PROBE = os.path.join(PKG, "calib", "mfma_probe")


def build_probe(verbose: bool = False) -> str:
    """Compile the standalone matrix-core calibration program (not part of the
    library); returns its path."""
    cmd = [hipcc(), *[f for f in COMMON_FLAGS if not f.startswith("-I") and f not in ("-fPIC", "-Wall")],
           PROBE_SRC, "-o", PROBE + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for mfma_probe.hip:\n{res.stdout}\n{res.stderr}")
    os.replace(PROBE + ".tmp", PROBE)
    return PROBE


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every HIP source and link libmiattn.so (and the calibration
    program); returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError(f"no HIP sources in {CSRC}")
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, s, o, verbose) for s, o in zip(srcs, objs)]
        for f in cf.as_completed(futs):
            src, dt = f.result()
            if verbose:
                print(f"compiled {os.path.basename(src)} in {dt:.1f}s", flush=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    build_probe(verbose)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    t0 = time.time()
    path = build(args.jobs, args.verbose)
    print(f"built {path} in {time.time() - t0:.1f}s")
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
