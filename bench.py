#!/usr/bin/env python3
"""Throughput of the fused-epilogue GEMM on one MI355X.

Headline workload: C = GELU(A.B + bias), A, B 2048 x 2048 fp16 (N(0,1)/sqrt(2048)),
bias[2048] fp16 N(0,1), erf-form GELU, fp16 output; fp32 accumulation on the
matrix cores.  One step = one launch of the fused kernel over one batch of
resident inputs (the whole hot path: tile mapping, pipelined operand staging,
MFMA main loop, register epilogue, single write of C).

Timing: W eager warmup launches, then K launches captured in one HIP graph,
which is replayed untimed until --warm-s seconds of wall time have passed
(default 1 s: the GPU clocks ramp up under sustained load, and timing right
after a short warmup under-reports the steady state), then the timed region:
one more replay of the K-launch graph between torch.cuda.synchronize()
calls.  HIP events recorded on the launch stream around the same replay give
the kernel's average duration for the roofline.  The JSON line records the
warm-up actually spent ("warm_s").  Inputs stay resident in HBM, so repeated
launches see warm L2/MALL, as in the pages' warmup-then-average method.

Prints ONE JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X dense matrix peaks and HBM bandwidth (published); 2516.6 = 256 CU x
# 4096 fp16 FLOP/clk/CU x 2.4 GHz, i.e. the published 2.5 PFLOP/s.
PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6}
PEAK_HBM_GBS = 8000.0
# MI355X's last-level cache (Infinity Cache / MALL) in front of HBM: a
# workload whose whole working set fits is served from it on repeated
# launches, so its rate is not an HBM rate.
MALL_BYTES = 256 << 20


def bandwidth_fields(nbytes: int, gbs: float) -> dict:
    """The rate of a bandwidth-bound workload against the HBM peak, labelled
    with the memory level that serves it: a working set that fits the MALL
    reports `pct_hbm_peak_mall_resident` (context, not an HBM figure)."""
    level = "mall" if nbytes <= MALL_BYTES else "hbm"
    key = "pct_hbm_peak" if level == "hbm" else "pct_hbm_peak_mall_resident"
    return {"GB/s": round(gbs, 1), "memory_level": level, key: round(100 * gbs / PEAK_HBM_GBS, 2)}


HEADLINE = "C3"
_CSRC = "dense_gemm_epilogues_tiled_amd/csrc/"
# The sources each workload's kernel is built from: counter readings taken on
# other sources are stale.
KERNEL_SOURCES = {
    "gemm": [_CSRC + "gemm.hip", _CSRC + "gemm_common.hpp", _CSRC + "device.hpp", _CSRC + "softmax.hip",
             _CSRC + "config_table.inc"],
    "stream": [_CSRC + "stream.hip", _CSRC + "device.hpp"],
    "attention": [_CSRC + "attention.hip", _CSRC + "device.hpp"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_family(workload: str) -> str:
    import workloads
    if workload in workloads.STREAM_WORKLOADS:
        return "stream"
    return "attention" if workload in workloads.ATTN_WORKLOADS else "gemm"


def kernel_source_sha(family: str = "gemm") -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha") != kernel_source_sha(kernel_family(workload)):
        return None
    return d.get("bytes_per_launch")


def warm_by_wall_time(replay, sync, seconds: float, batch: int = 8):
    """Replay `batch` times, synchronise, and repeat until `seconds` of wall
    time have passed (at least one batch).  Keeps the GPU busy so its clocks
    reach the level they hold under sustained load before anything is timed.
    Returns (replays, seconds spent)."""
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(batch):
            replay()
            n += 1
        sync()
        spent = time.perf_counter() - t0
        if spent >= seconds:
            return n, spent


def time_launches(launch, steps: int, warmup: int, stream, warm_s: float = 0.0, torch_mod=None):
    """Time `steps` launches.  `warmup` eager launches, then the `steps`
    launches are captured in one HIP graph, which is replayed untimed until
    `warm_s` seconds of wall time have passed (at least once: that also
    uploads it), then replayed once more between synchronisations (wall
    clock) and HIP events recorded on the launch stream (kernel time).
    Returns (wall ms per launch, event ms per launch, warm-up seconds)."""
    torch = torch_mod
    if torch is None:
        import torch
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            launch()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(steps):
            launch()

    def replay():
        with torch.cuda.stream(stream):
            g.replay()

    # a long graph needs few replays per synchronisation; a short one more, so
    # the queue stays ahead of the GPU
    _, warm_spent = warm_by_wall_time(replay, torch.cuda.synchronize, warm_s, batch=max(1, min(64, 2000 // steps)))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record(stream)
        g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps, e0.elapsed_time(e1) / steps, warm_spent


def kernel_name(cfg: dict) -> str:
    """The kernel a tile configuration launches."""
    import dense_gemm_epilogues_tiled_amd as tg
    if cfg["kind"] == tg.TG_KERNEL_GEMM_SOFTMAX:
        # the LDS-staged variants are built for column-major B only
        return "gemm_softmax_lds_kernel" if cfg["b_col_major"] == 1 else "gemm_softmax_kernel"
    return "gemm_ksplit_kernel" if cfg["waves"] == 2 * cfg["wave_m"] * cfg["wave_n"] else "gemm_tile_kernel"


def prepare(w, dev):
    import workloads
    A, B, bias = workloads.make_inputs(w)
    return A, B, bias, A.to(dev), B.to(dev), (bias.to(dev) if bias is not None else None)


def cpu_baseline(w, A, B, bias, min_seconds: float = 10.0, max_reps: int = 200):
    """The oracle on the full problem, repeated until `min_seconds` of wall
    time have passed (a bounded sample of ~10 s of CPU work), mean rate."""
    import oracle
    threads = oracle.default_threads()
    used = oracle.threads_used(threads)
    reps = 0
    t0 = time.perf_counter()
    while reps < max_reps and (reps == 0 or time.perf_counter() - t0 < min_seconds):
        oracle.gemm(A, B, bias, w.M, w.N, w.K, w.dtype, w.epilogue, b_col_major=w.b_col_major, alpha=w.alpha,
                    threads=threads)
        reps += 1
    dt = (time.perf_counter() - t0) / reps
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": w.flops / dt / 1e12, "unit": "TFLOP/s", "cores": used, "kind": "oracle",
            "sample": f"the full {w.M}x{w.N}x{w.K} problem {reps} times (fp64 triple loop + epilogue, OpenMP over "
                      f"rows), mean time per problem",
            "seconds": dt, "repetitions": reps, "cpu_model": cpu_model}


def bandwidth_table(dev, stream, names=None, steps=None, warmup: int = 10) -> dict:
    """The two bandwidth-bound kernels (vector addition and the standalone row
    softmax) on their seeded workloads: algorithmic bytes (inputs read once,
    outputs written once) per event-timed launch, against the HBM peak."""
    import torch

    import dense_gemm_epilogues_tiled_amd as tg
    import workloads
    table = {}
    for name, w in workloads.STREAM_WORKLOADS.items():
        if names is not None and name not in names:
            continue
        try:
            a, b = workloads.make_stream_inputs(w)
            ad = a.to(dev)
            bd = b.to(dev) if b is not None else None
            if w.kind == "vector_add":
                out = torch.empty_like(ad)

                def launch(ad=ad, bd=bd, out=out):
                    tg.vector_add(ad, bd, out=out)
            else:
                out = torch.empty((w.rows, w.cols), dtype=torch.float32, device=dev)

                def launch(ad=ad, w=w, out=out):
                    tg.row_softmax(ad, alpha=w.alpha, out=out)
            n = steps or (20 if w.min_bytes() > (1 << 30) else 100)
            wall, ev, _ = time_launches(launch, n, warmup, stream, warm_s=0.15)
            gbs = w.min_bytes() / (ev * 1e-3) / 1e9
            table[name] = {"kernel": "vector_add_kernel" if w.kind == "vector_add" else "row_softmax_kernel",
                           "workload": w.description, "us": round(ev * 1e3, 3), "us_wall": round(wall * 1e3, 3),
                           "algorithmic_bytes": w.min_bytes(), **bandwidth_fields(w.min_bytes(), gbs),
                           "traffic": measured_traffic(name)}
            log(f"  {name}: {table[name]}")
            del a, b, ad, bd, out
        except Exception as e:  # keep going: one failing workload must not hide the others
            table[name] = {"status": f"error: {e}"}
            log(f"  {name}: error {e}")
    return table


def attention_table(dev, stream, names=None, steps=None, warmup: int = 5) -> dict:
    """FlashAttention forward on its seeded workloads: 4 D FLOPs per visible
    (query, key) pair per event-timed launch, against the MFMA peak."""
    import torch

    import dense_gemm_epilogues_tiled_amd as tg
    import workloads
    table = {}
    for name, w in workloads.ATTN_WORKLOADS.items():
        if names is not None and name not in names:
            continue
        try:
            q, k, v = (t.to(dev) for t in workloads.make_attention_inputs(w))
            out = torch.empty_like(q)

            def launch(q=q, k=k, v=v, w=w, out=out):
                tg.attention(q, k, v, causal=w.causal, scale=w.scale, out=out)
            # long-running compute-bound kernel: give the clocks a full second
            wall, ev, _ = time_launches(launch, steps or 20, warmup, stream, warm_s=1.0)
            tf = w.flops / (ev * 1e-3) / 1e12
            table[name] = {"kernel": "attention_fwd_kernel", "workload": w.description, "us": round(ev * 1e3, 3),
                           "us_wall": round(wall * 1e3, 3), "algorithmic_flops": w.flops, "TFLOP/s": round(tf, 1),
                           "pct_mfma_peak": round(100 * tf / PEAK_TFLOPS[w.dtype], 2),
                           "traffic": measured_traffic(name)}
            log(f"  {name}: {table[name]}")
            del q, k, v, out
        except Exception as e:  # keep going: one failing workload must not hide the others
            table[name] = {"status": f"error: {e}"}
            log(f"  {name}: error {e}")
    return table


def build_parser() -> argparse.ArgumentParser:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=2000,
                    help="untimed eager launches before the graph is captured")
    ap.add_argument("--warm-s", type=float, default=1.0,
                    help="seconds of untimed graph replays right before the timed replay (the GPU clocks settle "
                         "under sustained load)")
    ap.add_argument("--workload", default=HEADLINE,
                    help="GEMM workload to time (default: the headline); a bandwidth (V1, V2, S1) or attention "
                         "(A1, A2, A3) workload name times that kernel alone and prints its entry (for profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-table", action="store_true", help="skip timing the other workloads")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before timing, copy a MIB-sized buffer 3 times (a plain copy kernel of known size "
                         "whose FETCH_SIZE / WRITE_SIZE counters calibrate HBM traffic readings)")
    return ap


def main() -> int:
    args = build_parser().parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("this benchmark runs on one GPU only (--gpus 1): the fused GEMM is measured on one GPU's "
               "share of the work, and no multi-GPU path exists")
        if int(os.environ.get("RANK", "0")) == 0:
            print(msg, file=sys.stderr)
        return 2

    import torch

    import dense_gemm_epilogues_tiled_amd as tg
    import workloads

    tg.load(build_if_missing=False)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name} ({getattr(props, 'gcnArchName', '?')}), {props.multi_processor_count} CUs")

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 copies of {args.copy_calibration} MiB")
        del src, dst

    if args.workload in workloads.STREAM_WORKLOADS:
        # one bandwidth-bound kernel alone (for profiling runs): its table entry
        t = bandwidth_table(dev, stream, [args.workload], args.steps, args.warmup)
        print(json.dumps({"name": args.workload, **t[args.workload]}), flush=True)
        return 0 if "status" not in t[args.workload] else 1

    if args.workload in workloads.ATTN_WORKLOADS:
        # the attention forward alone (for profiling runs): its table entry
        t = attention_table(dev, stream, [args.workload], args.steps, args.warmup)
        print(json.dumps({"name": args.workload, **t[args.workload]}), flush=True)
        return 0 if "status" not in t[args.workload] else 1

    w = workloads.WORKLOADS[args.workload]
    A, B, bias, Ad, Bd, bd = prepare(w, dev)
    out_dtype = torch.float32 if w.epilogue == "softmax" else Ad.dtype
    Cd = torch.empty((w.M, w.N), dtype=out_dtype, device=dev)

    def launch():
        tg.gemm(Ad, Bd, bd, epilogue=w.epilogue, b_col_major=w.b_col_major, alpha=w.alpha, out=Cd)

    log(f"timing {w.name}: {w.description}; warmup {args.warmup}, steps {args.steps}")
    ms_wall, ms_kernel, warm_spent = time_launches(launch, args.steps, args.warmup, stream, warm_s=args.warm_s)
    tflops = w.flops / (ms_wall * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    achieved = w.flops / (ms_kernel * 1e-3) / 1e12
    cfg = tg.query_config(w.M, w.N, w.K, Ad.dtype, w.epilogue, w.b_col_major)
    log(f"{w.name}: {ms_wall * 1e3:.2f} us/launch wall, {ms_kernel * 1e3:.2f} us/launch events, "
        f"{tflops:.1f} TFLOP/s ({100 * tflops / peak:.1f}% of {peak} TFLOP/s)")

    traffic = measured_traffic(w.name)
    # the shader clock under sustained MFMA load, right after the timed region
    clk = tg.shader_clock_mhz(dev)
    log(f"shader clock under MFMA load: {clk['mhz']:.0f} MHz "
        f"(dense fp16 MFMA peak at that clock {clk['peak_tflops_at_clock']:.1f} TFLOP/s)")
    result = {
        "metric": "TFLOP/s and % of MFMA peak, fp16 GEMM 2048^3 with fused bias+GELU",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warm_s": round(warm_spent, 3),
        "ms_per_step": ms_wall,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if w.dtype == "f16" else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.description}", "M": w.M, "N": w.N, "K": w.K,
                   "epilogue": w.epilogue, "accumulate": "f32", "tile_config": cfg},
        "pct_of_peak": round(100 * tflops / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel_us": round(ms_kernel * 1e3, 3), "algorithmic_flops_per_launch": w.flops,
                     "kernel": kernel_name(cfg),
                     "clock_mhz_under_mfma_load": round(clk["mhz"], 1),
                     "peak_at_measured_clock": round(clk["peak_tflops_at_clock"], 1),
                     "frac_at_measured_clock": round(achieved / clk["peak_tflops_at_clock"], 4)},
    }

    if not args.no_table:
        table = {}
        for name, wt in workloads.WORKLOADS.items():
            try:
                _, _, _, At, Bt, bt = prepare(wt, dev)
                od = torch.float32 if wt.epilogue == "softmax" else At.dtype
                Ct = torch.empty((wt.M, wt.N), dtype=od, device=dev)

                def lt(wt=wt, At=At, Bt=Bt, bt=bt, Ct=Ct):
                    tg.gemm(At, Bt, bt, epilogue=wt.epilogue, b_col_major=wt.b_col_major, alpha=wt.alpha, out=Ct)

                n = 50 if wt.M * wt.N * wt.K > 2 ** 36 else 1000
                wall, ev, _ = time_launches(lt, n, 10, stream, warm_s=args.warm_s)
                tf = wt.flops / (ev * 1e-3) / 1e12
                gbs = wt.min_bytes() / (ev * 1e-3) / 1e9
                table[name] = {"us": round(ev * 1e3, 3), "us_wall": round(wall * 1e3, 3), "TFLOP/s": round(tf, 1),
                               "pct_mfma_peak": round(100 * tf / PEAK_TFLOPS[wt.dtype], 2),
                               "GB/s": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
                               "tile_config": tg.query_config(wt.M, wt.N, wt.K, At.dtype, wt.epilogue,
                                                              wt.b_col_major)["id"]}
                log(f"  {name}: {table[name]}")
                del At, Bt, bt, Ct
            except Exception as e:  # keep going: one failing workload must not hide the others
                table[name] = {"status": f"error: {e}"}
                log(f"  {name}: error {e}")
        result["workloads"] = table
        result["bandwidth"] = bandwidth_table(dev, stream)
        result["attention"] = attention_table(dev, stream)

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the same workload ...")
        result["cpu_baseline"] = cpu_baseline(w, A, B, bias)
        log(f"cpu_baseline: {result['cpu_baseline']}")
    result["host"] = {"python": platform.python_version(), "torch": torch.__version__,
                      "hip": getattr(torch.version, "hip", None), "gpu": props.name}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
