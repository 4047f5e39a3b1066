"""Build the HGA HIP library (gfx950) in-tree: long_context_hga_amd/libhga.so."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libhga.so")
CALIB = os.path.join(PKG, "calib")
CALIB_OUT = os.path.join(PKG, "libhga_calib.so")
BUILD = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        err = "\n".join(l for l in r.stderr.splitlines()
                        if "packed-fp32-ops" not in l)  # host pass does not know the feature
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = OUT + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, OUT)
    # the benchmark's calibration kernels (not part of the HGA path: a
    # failure here is reported and leaves the library build standing)
    tmp = CALIB_OUT + ".tmp"
    r = subprocess.run([HIPCC, *FLAGS, "-shared", "-o", tmp, *sorted(glob.glob(os.path.join(CALIB, "*.hip")))],
                       capture_output=True, text=True)
    if r.returncode != 0:
        print(f"warning: hipcc failed for the calibration kernels (bench.py --calibrate-mfma "
              f"unavailable):\n{r.stderr}", file=sys.stderr)
    else:
        os.replace(tmp, CALIB_OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
