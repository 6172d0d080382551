"""Build libtg.so (the gfx950 kernels and the C ABI of include/tg.h) in-tree.

    python -m dense_gemm_epilogues_tiled_amd.build

Compiles every source in csrc/ with hipcc for gfx950 only and links one
shared library next to this file.  Packed-fp32 instruction selection is
disabled on the device side (-Xclang -target-feature -Xclang -packed-fp32-ops);
hipcc's host pass warns that it does not know that feature, which is harmless.

Every compile also asks for the compiler's per-kernel resource report
(-Rpass-analysis=kernel-resource-usage): registers, scratch (spill) bytes
per lane, LDS and occupancy of each kernel.  The reports are collected into
_build/kernel_resources.json; `--report PATH` also writes them as a text
table.  A kernel that needs scratch memory spills registers to memory, which
the kernels here are built never to do (tests/test_resources.py checks it).
"""

from __future__ import annotations

import json
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libtg.so")
BUILD_DIR = os.path.join(HERE, "_build")
RESOURCES = os.path.join(BUILD_DIR, "kernel_resources.json")

SOURCES = ["gemm.hip", "softmax.hip", "stream.hip", "attention.hip", "autotune.hip", "clock.hip", "layout.hip",
           "api.cpp", "autotune_cache.cpp"]
# The sources that hold host code only (argument checks, configuration
# lookup, the autotune cache and its file format): the CPU sanitizer run
# builds these with AddressSanitizer and UndefinedBehaviorSanitizer.
HOST_SOURCES = ["api.cpp", "autotune_cache.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
    # '#pragma unroll' on the store loops whose start is the thread id: the
    # trip count is not constant, the loop stays rolled, as intended
    "-Wno-pass-failed",
]
REMARK_FLAG = "-Rpass-analysis=kernel-resource-usage"

# "<file>:<line>:<col>: remark: <key>: <value> [-Rpass-analysis=kernel-resource-usage]"
_REMARK = re.compile(r"remark:\s+(?P<key>[^:]+?):\s+(?P<val>.*?)\s+\[-Rpass-analysis=kernel-resource-usage\]")
_FIELDS = {"TotalSGPRs": "sgprs", "VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch_bytes",
           "Dynamic Stack": "dynamic_stack", "Occupancy [waves/SIMD]": "occupancy", "SGPRs Spill": "sgpr_spill",
           "VGPRs Spill": "vgpr_spill", "LDS Size [bytes/block]": "lds_bytes"}


def parse_resource_remarks(text: str) -> dict:
    """Per-kernel resource fields from the compiler's kernel-resource-usage
    remarks: {mangled kernel name: {field: int or bool}}."""
    out, cur = {}, None
    for line in text.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group("key").strip(), m.group("val").strip()
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None and key in _FIELDS:
            cur[_FIELDS[key]] = (val == "True") if val in ("True", "False") else int(val)
    return out


def demangle(names):
    """Readable kernel names (c++filt from binutils); unchanged if it is missing."""
    for tool in ("c++filt", "/opt/rocm/llvm/bin/llvm-cxxfilt"):
        try:
            r = subprocess.run([tool], input="\n".join(names), capture_output=True, text=True, check=True)
        except (OSError, subprocess.CalledProcessError):
            continue
        out = r.stdout.splitlines()
        if len(out) == len(names):
            return dict(zip(names, out))
    return {n: n for n in names}


def _compile(src: str, build_dir: str = BUILD_DIR, defines=()):
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *(f"-D{d}" for d in defines), REMARK_FLAG, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    text = r.stdout + r.stderr
    noise = "is not a recognized feature for this target"
    # keep warnings and errors, drop the resource remarks and their source excerpts
    lines, skip = [], 0
    for l in text.splitlines():
        if skip:
            skip -= 1
            continue
        if "kernel-resource-usage" in l:
            if "Function Name" in l:
                skip = 2  # the quoted source line and the caret under it
            continue
        if noise in l:
            continue
        lines.append(l)
    msg = "\n".join(lines)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip():
        sys.stderr.write(msg + "\n")
    return obj, {name: dict(f, source=src) for name, f in parse_resource_remarks(text).items()}


def write_report(resources: dict, path: str) -> None:
    """The per-kernel resource table as text."""
    rows = sorted(resources.items(), key=lambda kv: (kv[1]["source"], kv[1].get("demangled", kv[0])))
    with open(path, "w") as f:
        f.write("Per-kernel resources of libtg.so, from the compiler's kernel-resource-usage report\n")
        f.write("(hipcc --offload-arch=gfx950 -O3 " + REMARK_FLAG + "; written by\n")
        f.write(" python -m dense_gemm_epilogues_tiled_amd.build --report profiles/kernel_resources.txt).\n")
        f.write("VGPR/AGPR: registers per lane; scratch: spill bytes per lane; occ: waves per SIMD.\n\n")
        f.write(f"{'VGPR':>5} {'AGPR':>5} {'SGPR':>5} {'scratch':>7} {'LDS':>7} {'occ':>4}  kernel\n")
        for name, r in rows:
            f.write(f"{r.get('vgprs', -1):>5} {r.get('agprs', -1):>5} {r.get('sgprs', -1):>5} "
                    f"{r.get('scratch_bytes', -1):>7} {r.get('lds_bytes', -1):>7} {r.get('occupancy', -1):>4}  "
                    f"{r.get('demangled', name)}\n")


def build(verbose: bool = False, report: str | None = None, defines=(), out: str = OUT,
          build_dir: str = BUILD_DIR) -> str:
    """Compile and link.  `defines` (e.g. TG_PHASE_STAMPS for the profiling
    build) go to every compile; such builds should name their own `out` and
    `build_dir` so the product library and its objects stay as they are."""
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        done = list(ex.map(lambda src: _compile(src, build_dir, defines), SOURCES))
    objs = [o for o, _ in done]
    resources = {}
    for _, res in done:
        resources.update(res)
    for name, full in demangle(sorted(resources)).items():
        resources[name]["demangled"] = full
    with open(os.path.join(build_dir, os.path.basename(RESOURCES)), "w") as f:
        json.dump(resources, f, indent=1, sort_keys=True)
    if report:
        write_report(resources, report)
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--report", metavar="PATH", help="also write the per-kernel resource table as text")
    build(verbose=True, report=ap.parse_args().report)
