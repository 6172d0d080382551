"""Offline tile-configuration sweep: validate, time, bake the winners.

    python -m dense_gemm_epilogues_tiled_amd.sweep [--workloads C2,C3,...] [--write-table]

The TileLang pages pick tile shapes, warp counts and pipeline depth per
matrix shape by search ("Exploracao de schedules com autotuning",
noticiai.com.br: search space over tile sizes and warp counts keyed on
(M, N, K), results cached; the spaxe.top page: schedules over the shared
memory budget are skipped, each candidate is checked, the autotuned choice
matches the best hand-picked one).  Here the search runs offline on the
target GPU over the compiled variants of libtg.so (each already within the
160 KB LDS budget) and over the raster band height and XCD regrouping:

  0. candidates whose kernel needs scratch memory (register spills, from the
     build's kernel-resource report, _build/kernel_resources.json) are
     skipped;
  1. every candidate runs once and is compared with an fp32 reference of
     the same inputs computed by torch on the GPU (the acceptance bound:
     1e-2 + 1e-2|ref| per element, 2e-3 relative Frobenius; 1e-4 for the fp32
     softmax output) -- a failing candidate is never timed;
  2. surviving candidates are timed with a HIP graph of back-to-back launches;
  3. the fastest per shape is written to csrc/config_table.inc
     (--write-table), after which the library must be rebuilt.

Results go to a JSON file (--results, by default in the system's temporary
directory) so an interrupted sweep can resume; the file records the hash of
the kernel sources, and rows measured on other sources are discarded.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import tempfile
import time

import torch

import dense_gemm_epilogues_tiled_amd as tg

HERE = os.path.dirname(os.path.abspath(__file__))
TABLE = os.path.join(HERE, "csrc", "config_table.inc")
ROOT = os.path.dirname(HERE)
DEFAULT_RESULTS = os.path.join(tempfile.gettempdir(), "tg_sweep_results.json")
# the sources the compiled variants are built from (not the table itself)
KERNEL_SOURCES = ["gemm.hip", "gemm_common.hpp", "device.hpp", "softmax.hip", "kernels.hpp"]


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(HERE, "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_prefix(cfg: dict) -> str:
    """The start of the demangled name of every kernel instance a tile
    configuration may launch (all dtypes, B layouts and schedule orders)."""
    if cfg["kind"] == tg.TG_KERNEL_GEMM_SOFTMAX:
        s = cfg["bn"] // (16 * cfg["waves"])
        if cfg["b_col_major"] == 1:
            return f"void tg::gemm_softmax_lds_kernel<{cfg['waves']}, {s}, {'true' if cfg['bk'] == 64 else 'false'}, "
        return f"void tg::gemm_softmax_kernel<{cfg['waves']}, {s}, {cfg['bk'] // 32}, "
    if cfg["waves"] == 2 * cfg["wave_m"] * cfg["wave_n"]:
        return f"void tg::gemm_ksplit_kernel<{cfg['bm']}, {cfg['bn']}, {cfg['wave_m']}, {cfg['wave_n']}, {cfg['stages']}, "
    return (f"void tg::gemm_tile_kernel<{cfg['bm']}, {cfg['bn']}, {cfg['bk']}, {cfg['wave_m']}, {cfg['wave_n']}, "
            f"{cfg['stages']}, ")


def spilling_configs(resources: dict, configs) -> set:
    """Ids of the configurations whose kernels (any instance) need scratch
    memory, from the build's {mangled name: {demangled, scratch_bytes, ...}}."""
    bad = set()
    for c in configs:
        pre = kernel_prefix(c)
        for r in resources.values():
            if r.get("demangled", "").startswith(pre) and (r.get("scratch_bytes", 0) or r.get("vgpr_spill", 0)):
                bad.add(c["id"])
    return bad


def load_results(path: str | None) -> dict:
    """Rows of an earlier run on the same kernel sources, else nothing."""
    if not path or not os.path.exists(path):
        return {}
    with open(path) as f:
        d = json.load(f)
    if not isinstance(d, dict) or d.get("kernel_source_sha") != kernel_source_sha():
        return {}
    return d.get("workloads", {})


def _workloads():
    sys.path.insert(0, ROOT)
    import workloads
    return workloads


def reference(A, B, bias, epilogue, b_col_major, alpha):
    """fp32 reference on the GPU: torch matmul of the exact fp16/bf16 inputs."""
    Bm = B.float().t().contiguous() if b_col_major else B.float()
    x = alpha * (A.float() @ Bm)
    if bias is not None:
        x = x + bias.float()
    if epilogue == "relu":
        return torch.relu(x)
    if epilogue == "gelu":
        return torch.nn.functional.gelu(x, approximate="none")
    if epilogue == "softmax":
        return torch.softmax(x, dim=1)
    return x


def check(C, ref, out_f32):
    atol = rtol = 1e-4 if out_f32 else 1e-2
    g = C.float()
    err = (g - ref).abs()
    ok = bool(torch.isfinite(g).all()) and bool((err <= atol + rtol * ref.abs()).all())
    frob = float(torch.linalg.vector_norm(g - ref) / torch.linalg.vector_norm(ref))
    return ok and frob <= 2e-3, frob


def time_graph(fn, n, stream):
    with torch.cuda.stream(stream):
        for _ in range(5):
            fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(n):
            fn()
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = float("inf")
    for _ in range(3):
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e3 / n)
    return best  # microseconds per launch


def candidates(kind):
    out = []
    for c in tg.configs():
        if c["kind"] != kind:
            continue
        if kind == tg.TG_KERNEL_GEMM:
            for gm in (1, 2, 4, 8, 16):
                for xcd in (0, 1):
                    out.append((c["id"], gm, xcd))
        else:
            out.append((c["id"], 1, 0))
    return out


def sweep(names, results_path, stream, log=print):
    W = _workloads()
    results = load_results(results_path)
    res_file = os.path.join(HERE, "_build", "kernel_resources.json")
    skip = set()
    if os.path.exists(res_file):
        with open(res_file) as f:
            skip = spilling_configs(json.load(f), tg.configs())
    if skip:
        log(f"skipping configurations whose kernels spill: {sorted(skip)}")
    dev = torch.device("cuda:0")
    for name in names:
        w = W.WORKLOADS[name]
        A, B, bias = W.make_inputs(w)
        Ad, Bd = A.to(dev), B.to(dev)
        bd = bias.to(dev) if bias is not None else None
        ref = reference(Ad, Bd, bd, w.epilogue, w.b_col_major, w.alpha)
        out_f32 = w.epilogue == "softmax"
        C = torch.empty((w.M, w.N), dtype=torch.float32 if out_f32 else Ad.dtype, device=dev)
        kind = tg.TG_KERNEL_GEMM_SOFTMAX if out_f32 else tg.TG_KERNEL_GEMM
        # long graphs: in graphs of a few hundred launches a short kernel's
        # dispatches were measured ~2.5 us longer than in graphs of 1000+
        n = 20 if w.flops > 2 ** 38 else 1000
        # let the clocks ramp up under load before the first candidate
        t_warm = time.time() + 0.5
        while time.time() < t_warm:
            tg.gemm(Ad, Bd, bd, epilogue=w.epilogue, b_col_major=w.b_col_major, alpha=w.alpha, out=C)
            torch.cuda.synchronize()
        rows = results.setdefault(name, {})
        for cid, gm, xcd in candidates(kind):
            key = f"{cid}/{gm}/{xcd}"
            if key in rows or cid in skip:
                continue
            cfg = tg.configs()[cid]
            if kind == tg.TG_KERNEL_GEMM_SOFTMAX and cfg["bn"] < w.N:
                continue

            def launch(cid=cid, gm=gm, xcd=xcd):
                tg.gemm(Ad, Bd, bd, epilogue=w.epilogue, b_col_major=w.b_col_major, alpha=w.alpha, out=C,
                        config_id=cid, group_m=gm, xcd_remap=xcd)

            C.fill_(float("nan"))
            launch()
            torch.cuda.synchronize()
            ok, frob = check(C, ref, out_f32)
            rec = {"id": cid, "group_m": gm, "xcd_remap": xcd, "valid": ok, "frob": frob}
            if ok:
                us = time_graph(launch, n, stream)
                rec.update({"us": us, "tflops": w.flops / us / 1e6})
            rows[key] = rec
            log(f"{name} cfg {cid} ({cfg['bm']}x{cfg['bn']}x{cfg['bk']} st{cfg['stages']} w{cfg['waves']}) "
                f"group_m {gm} xcd {xcd}: " + (f"{rec['us']:.2f} us {rec['tflops']:.1f} TFLOP/s" if ok else
                                               f"INVALID (frob {frob:.2e})"))
            if results_path:
                with open(results_path, "w") as f:
                    json.dump({"kernel_source_sha": kernel_source_sha(), "workloads": results}, f, indent=1)
        del Ad, Bd, bd, ref, C
    return results


def best_per_workload(results):
    best = {}
    for name, rows in results.items():
        valid = [r for r in rows.values() if r.get("valid") and "us" in r]
        if valid:
            best[name] = min(valid, key=lambda r: r["us"])
    return best


def write_table(best, path=TABLE):
    W = _workloads()
    lines = [
        "// config_table.inc -- per-shape tile choices baked into the library.",
        "// Written by dense_gemm_epilogues_tiled_amd/sweep.py: for each shape the fastest",
        "// candidate among those that matched the fp32 reference, timed on an MI355X.",
        "// Fields: dtype, b_col_major, epilogue kind (0 elementwise, 1 softmax), M, N, K,",
        "//         configuration id, group_m, xcd_remap.",
        "static const TableEntry kTable[] = {",
    ]
    seen = set()
    # when two workloads share a table key (same dtype, layout, kind and shape),
    # the headline one decides: the fused bias+GELU 2048^3 case before plain 2048^3
    priority = ["C3", "C2", "C4a", "C4b", "C5", "C1"]
    order = sorted(best, key=lambda n: (priority.index(n) if n in priority else len(priority), n))
    for name in order:
        r = best[name]
        w = W.WORKLOADS[name]
        dt = "TG_DTYPE_F16" if w.dtype == "f16" else "TG_DTYPE_BF16"
        kind = 1 if w.epilogue == "softmax" else 0
        key = (dt, int(w.b_col_major), kind, w.M, w.N, w.K)
        if key in seen:
            continue
        seen.add(key)
        lines.append(f"    {{{dt}, {int(w.b_col_major)}, {kind}, {w.M}, {w.N}, {w.K}, {r['id']}, {r['group_m']}, "
                     f"{r['xcd_remap']}}},  // {name}: {r['us']:.2f} us, {r['tflops']:.0f} TFLOP/s")
    lines.append("};")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workloads", default="C2,C3,C4a,C4b,C5")
    ap.add_argument("--results", default=DEFAULT_RESULTS,
                    help="JSON file of measured candidates, to resume an interrupted sweep (rows measured on other "
                         "kernel sources are discarded)")
    ap.add_argument("--write-table", action="store_true")
    args = ap.parse_args()
    tg.load(build_if_missing=False)
    stream = torch.cuda.Stream()
    t0 = time.time()
    res = sweep(args.workloads.split(","), args.results, stream, log=lambda s: print(s, flush=True))
    best = best_per_workload(res)
    for name, r in best.items():
        print(f"best {name}: {r}", flush=True)
    if args.write_table:
        write_table(best)
        print(f"wrote {TABLE}", flush=True)
    print(f"sweep took {time.time() - t0:.1f} s", flush=True)


if __name__ == "__main__":
    main()
