"""HBM traffic per launch from rocprofv3 counter passes.

    python -m dense_gemm_epilogues_tiled_amd.traffic <workload> <fetch_dir> <write_dir>

Each directory holds the output of one counter pass over bench.py timing one
workload alone, with a plain device copy of known size first:

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch_dir> -o p -- \\
        python3 bench.py --workload <W> --steps 10 --warmup 2 --no-cpu-baseline --no-table --copy-calibration 256
    rocprofv3 --pmc WRITE_SIZE ...  (same, into <write_dir>)

FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch (summed over the L2
channels).  The copy moves 256 MiB each way, so its readings give the factor
from counter units to bytes for each counter; the workload kernel's median
reading times that factor is its HBM traffic per launch.  The result goes to
profiles/hbm_traffic_<W>.json with the hash of the kernel's sources (bench.py
uses it only while the sources are unchanged), and the human-readable summary
profiles/hbm_traffic_counters.txt is rewritten from every such file.
"""

from __future__ import annotations

import csv
import glob
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PROFILES = os.path.join(ROOT, "profiles")
COPY_MIB = 256
KERNEL_PREFIX = {"gemm": ("gemm_tile_kernel", "gemm_ksplit_kernel", "gemm_softmax"), "stream": ("vector_add", "row_softmax"),
                 "attention": ("attention_fwd",)}


def read_counter(directory: str, counter: str) -> dict:
    """kernel name -> list of per-dispatch values (summed over instances)."""
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {directory}")
    per_dispatch = {}
    for path in files:
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                key = (path, row["Dispatch_Id"], row["Kernel_Name"])
                per_dispatch[key] = per_dispatch.get(key, 0.0) + float(row["Counter_Value"])
    out = {}
    for (_, _, name), v in per_dispatch.items():
        out.setdefault(name, []).append(v)
    return out


def pick(values: dict, prefixes) -> tuple[str, float]:
    names = [n for n in values if any(p in n for p in prefixes)]
    if not names:
        raise LookupError(f"no kernel matching {prefixes} in {sorted(values)}")
    name = max(names, key=lambda n: len(values[n]))
    return name, statistics.median(values[name])


def measure(workload: str, fetch_dir: str, write_dir: str) -> dict:
    """The traffic record of one workload from its two counter passes."""
    sys.path.insert(0, ROOT)
    import bench
    import workloads as W

    family = bench.kernel_family(workload)
    w = (W.WORKLOADS.get(workload) or W.STREAM_WORKLOADS.get(workload) or W.ATTN_WORKLOADS.get(workload))
    fetch = read_counter(fetch_dir, "FETCH_SIZE")
    write = read_counter(write_dir, "WRITE_SIZE")
    copy_kib = COPY_MIB * 1024
    _, copy_fetch = pick(fetch, ("copyBuffer", "copy"))
    _, copy_write = pick(write, ("copyBuffer", "copy"))
    kname, k_fetch = pick(fetch, KERNEL_PREFIX[family])
    _, k_write = pick(write, KERNEL_PREFIX[family])
    fetch_scale = copy_kib / copy_fetch
    write_scale = copy_kib / copy_write
    rec = {
        "kernel": kname,
        "fetch_bytes": k_fetch * fetch_scale * 1024,
        "write_bytes": k_write * write_scale * 1024,
        "algorithmic_bytes": w.min_bytes() if callable(w.min_bytes) else w.min_bytes,
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "kernel_source_sha": bench.kernel_source_sha(family),
        "source": "profiles/hbm_traffic_counters.txt",
    }
    rec["bytes_per_launch"] = rec["fetch_bytes"] + rec["write_bytes"]
    return rec


def summarize(workload: str, fetch_dir: str, write_dir: str) -> dict:
    """measure(), then write profiles/hbm_traffic_<workload>.json and the text summary."""
    rec = measure(workload, fetch_dir, write_dir)
    with open(os.path.join(PROFILES, f"hbm_traffic_{workload}.json"), "w") as f:
        json.dump(rec, f, indent=1)
    write_text()
    return rec


def write_text() -> None:
    sys.path.insert(0, ROOT)
    import workloads as W

    order = list(W.WORKLOADS) + list(W.STREAM_WORKLOADS) + list(W.ATTN_WORKLOADS)
    lines = [
        "HBM traffic per launch from rocprofv3 counters (KiB as reported, summed over all TCC instances),",
        f"scaled by a plain copy kernel of known size measured in the same run ({COPY_MIB} MiB device-to-device copy:",
        f"reads {COPY_MIB * 1024} KiB, writes {COPY_MIB * 1024} KiB).",
        "commands (one pass each), then python -m dense_gemm_epilogues_tiled_amd.traffic <W> <fetch out> <write out>:",
        "  cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch out> -o p -- python3 $REPO/bench.py "
        f"--workload <W> --steps 10 --warmup 2 --no-cpu-baseline --no-table --copy-calibration {COPY_MIB}",
        "  cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write out> -o p -- python3 $REPO/bench.py "
        f"--workload <W> --steps 10 --warmup 2 --no-cpu-baseline --no-table --copy-calibration {COPY_MIB}",
        "",
    ]
    mib = 1 << 20
    for name in order:
        path = os.path.join(PROFILES, f"hbm_traffic_{name}.json")
        if not os.path.exists(path):
            continue
        with open(path) as f:
            d = json.load(f)
        w = W.WORKLOADS.get(name) or W.STREAM_WORKLOADS.get(name) or W.ATTN_WORKLOADS.get(name)
        total = d["bytes_per_launch"]
        lines += [
            f"{name} ({w.description})",
            f"  kernel: {d['kernel']}",
            f"  kernel sources sha {d['kernel_source_sha']}",
            f"  scale factors (copy's true bytes / counter bytes): FETCH_SIZE x{d['fetch_scale']:.3f}, "
            f"WRITE_SIZE x{d['write_scale']:.3f}",
            f"  FETCH {d['fetch_bytes'] / mib:8.2f} MiB  WRITE {d['write_bytes'] / mib:8.2f} MiB  total "
            f"{total / mib:8.2f} MiB per launch; algorithmic {d['algorithmic_bytes'] / mib:.2f} MiB "
            f"(ratio {total / d['algorithmic_bytes']:.2f})",
        ]
    with open(os.path.join(PROFILES, "hbm_traffic_counters.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if len(sys.argv) != 4:
        sys.exit(__doc__)
    print(json.dumps(summarize(sys.argv[1], sys.argv[2], sys.argv[3]), indent=1))
