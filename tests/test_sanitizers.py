"""CPU: AddressSanitizer + UndefinedBehaviorSanitizer runs of the host code.

- The oracle (oracle/oracle.c), built with gcc and the sanitizers, driven by
  tests/sanitize/oracle_driver.c: every exported function on exact-size
  buffers over small shapes, empty and one-element cases included, and with
  invalid arguments.
- The library's host-only sources (build.HOST_SOURCES: argument checks,
  configuration lookup, the autotune cache and its file parser), built with
  the ROCm clang++ and the sanitizers, linked with the library's other
  objects from the in-tree build (uninstrumented; only their host launchers
  and variant tables are reached) and driven by tests/sanitize/abi_driver.c:
  configuration queries over a grid of shapes up to INT64_MAX, every entry
  point with invalid arguments, and the cache parser on well-formed and
  malformed files.  No call reaches the HIP runtime.

A sanitizer finding aborts the driver with a report; the test prints it.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ROCM_CLANG = "/opt/rocm/llvm/bin/clang"
ROCM_CLANGXX = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if r.returncode != 0:
        pytest.fail(f"{' '.join(cmd)} -> {r.returncode}\n{r.stdout[-4000:]}\n{r.stderr[-8000:]}")
    return r


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not installed")
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c99", "-fopenmp", "-ffp-contract=off", *SAN, "-fsanitize=float-cast-overflow",
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_driver.c"), "-lm", "-o", exe])
    r = _run([exe], env=dict(ENV, OMP_NUM_THREADS="2"), timeout=300)
    assert "oracle_driver: ok" in r.stdout


def _stale_objects(tg_build):
    """Objects of the in-tree build that are missing or older than what they
    are built from (their source, or any header)."""
    headers = [os.path.join(ROOT, "include", "tg.h")] + [
        os.path.join(tg_build.CSRC, f) for f in os.listdir(tg_build.CSRC) if f.endswith((".hpp", ".inc"))]
    newest_header = max(os.path.getmtime(h) for h in headers)
    stale = []
    for src in tg_build.SOURCES:
        obj = os.path.join(tg_build.BUILD_DIR, os.path.splitext(src)[0] + ".o")
        if (not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(os.path.join(tg_build.CSRC, src))
                or os.path.getmtime(obj) < newest_header):
            stale.append(os.path.basename(obj))
    return stale


def test_abi_host_code_under_sanitizers(tmp_path):
    from dense_gemm_epilogues_tiled_amd import build as tg_build
    if not (os.path.exists(ROCM_CLANG) and os.path.exists(ROCM_CLANGXX)):
        pytest.skip("the ROCm clang is not installed")
    stale = _stale_objects(tg_build)
    if stale:
        pytest.skip(f"the in-tree build is missing or older than its sources ({', '.join(stale)}): "
                    "run python -m dense_gemm_epilogues_tiled_amd.build")
    objs = []
    for src in tg_build.HOST_SOURCES:
        obj = str(tmp_path / ("san_" + os.path.splitext(src)[0] + ".o"))
        _run([ROCM_CLANGXX, "-std=c++20", "-fPIC", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
              "-I", os.path.join(ROOT, "include"), "-I", tg_build.CSRC, "-c", os.path.join(tg_build.CSRC, src),
              "-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "abi_driver.o")
    _run([ROCM_CLANG, "-std=c99", "-Wall", "-Werror", *SAN, "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(HERE, "abi_driver.c"), "-o", drv])
    product = [os.path.join(tg_build.BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in tg_build.SOURCES
               if s not in tg_build.HOST_SOURCES]
    exe = str(tmp_path / "abi_driver")
    _run([ROCM_CLANGXX, *SAN, drv, *objs, *product, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
          "-o", exe])
    scratch = tmp_path / "scratch"
    scratch.mkdir()
    r = _run([exe, str(scratch)], env=ENV, timeout=300)
    assert "abi_driver:" in r.stdout and r.stdout.strip().endswith("ok")
