"""AddressSanitizer + UndefinedBehaviorSanitizer runs on the CPU.

  * the fp64 oracle: every function driven once on small inputs
    (oracle/sanitize_check.c), built with gcc -fsanitize=address,undefined;
  * the library's host code: every entry point's argument checks and the
    configuration / size queries (tests/abi_sanitize_driver.c), with the HIP
    sources built by hipcc for gfx950 and the sanitizers applied to the host
    side only (-Xarch_host before each -fsanitize=).  Every call the driver
    makes is answered on the host, so no GPU is needed.
Both programs end with a sanitizer report (non-zero exit) on any
out-of-bounds access, use after free, leak or undefined operation."""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address", "-fsanitize=undefined"]


def _run(cmd, env=None, timeout=300):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=env)
    assert r.returncode == 0, (cmd, r.stdout[-3000:], r.stderr[-3000:])
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "sanitize_check")
    _run(["gcc", "-O1", "-g", *SAN, "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          "-fopenmp", os.path.join(ROOT, "oracle", "hga_oracle.c"),
          os.path.join(ROOT, "oracle", "sanitize_check.c"), "-lm", "-o", exe])
    env = dict(os.environ, OMP_NUM_THREADS="2")
    assert "sanitize ok" in _run([exe], env=env)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_library_host_code_under_asan_ubsan(tmp_path):
    csrc = os.path.join(ROOT, "long_context_hga_amd", "csrc")
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", "-Xclang",
             "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
             "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
             "-I" + os.path.join(ROOT, "include"), "-I" + csrc]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, *flags, "-c", src, "-o", obj], timeout=600)
        return obj

    srcs = sorted(glob.glob(os.path.join(csrc, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_san")
    _run([HIPCC, "--offload-arch=gfx950", "-g", *host_san, "-I" + os.path.join(ROOT, "include"),
          "-x", "c", os.path.join(ROOT, "tests", "abi_sanitize_driver.c"), "-x", "none", *objs,
          "-o", exe], timeout=600)
    assert "abi sanitize ok" in _run([exe])
