"""Phase breakdown of a workload's kernel from a profiling build.

    python -m dense_gemm_epilogues_tiled_amd.phases --build           (CPU: builds libtg_phases.so)
    python -m dense_gemm_epilogues_tiled_amd.phases C3 [C5 ...] [--config ID] [--steps N]   (GPU)

The profiling build compiles every source with -DTG_PHASE_STAMPS (see
csrc/phases.hpp): the instrumented kernels read the GPU's constant 100 MHz
clock at named points of their schedule and write the stamps of wave 0 of
every workgroup to a device array; the work itself is unchanged.  This tool
runs a workload the way bench.py times it (HIP graph of N launches after a
one-second warm-up), reads the stamps of the last launch and prints, per
phase, when the workgroups reached it, counted from the first workgroup's
start (min / median / max over workgroups, microseconds), and the median
time each phase took.  The HIP-event time per launch is printed beside it:
the difference to the stamped span is dispatch time outside the workgroups.
"""

from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libtg_phases.so")
BUILD_DIR = os.path.join(HERE, "_build_phases")
TICK_US = 0.01  # one tick of the 100 MHz constant clock

PHASES = {
    "gemm_ksplit_kernel": ["entry", "prologue copies issued", "first stage landed", "main loop done",
                           "partials exchanged", "first row round stored", "last row round stored",
                           "stores drained"],
    "gemm_tile_kernel": ["entry", "prologue copies issued", "first stage landed", "main loop done",
                         "activation done", "ring free", "stores issued", "stores drained"],
    "gemm_softmax_lds_kernel": ["entry", "first copies issued", "first step landed", "product done",
                                "wave pairs exchanged", "pairs combined", "stores issued", "stores drained"],
    # per pass over a query block (the causal kernel makes two per workgroup)
    "attention_fwd_kernel": ["pass 1 start", "pass 1 first block landed", "pass 1 last block done",
                             "pass 1 O stored", "pass 2 start", "pass 2 first block landed",
                             "pass 2 last block done", "pass 2 O stored"],
}
# the stamp array each kernel family writes (one per source file)
READER = {"gemm_ksplit_kernel": "tg_phases_gemm", "gemm_tile_kernel": "tg_phases_gemm",
          "gemm_softmax_lds_kernel": "tg_phases_softmax", "attention_fwd_kernel": "tg_phases_attention"}


def build_profiling_library() -> str:
    from . import build as tg_build
    return tg_build.build(verbose=True, defines=("TG_PHASE_STAMPS",), out=LIB, build_dir=BUILD_DIR)


def summarize(stamps: np.ndarray, names) -> list[str]:
    """stamps: groups x 8 ticks of the constant clock; a 0 is a phase the
    workgroup did not pass (e.g. the second pass of a one-pass workgroup)
    and rows of zeros are workgroups the launch did not have."""
    stamps = stamps[(stamps != 0).any(axis=1)]
    t = stamps.astype(np.float64)
    t[stamps == 0] = np.nan
    t = (t - np.nanmin(t[:, 0])) * TICK_US
    lines = [f"  {'phase':<26} {'min':>8} {'median':>8} {'max':>8}   median duration (us)   workgroups"]
    for i, name in enumerate(names):
        col = t[:, i]
        if np.isnan(col).all():
            continue
        dur = np.nanmedian(t[:, i] - t[:, i - 1]) if i > 0 and not np.isnan(t[:, i] - t[:, i - 1]).all() else 0.0
        lines.append(f"  {name:<26} {np.nanmin(col):8.3f} {np.nanmedian(col):8.3f} {np.nanmax(col):8.3f}   "
                     f"{dur:8.3f}   {int((~np.isnan(col)).sum()):10d}")
    lines.append(f"  span (first start to last stamp): {np.nanmax(t):.3f} us over {len(t)} workgroups")
    return lines


def attention_phases(name, lib, dev, stream, steps, bench, tg, workloads) -> None:
    """The attention kernel on one of its workloads: stamps per pass over a
    query block (one pass per workgroup, two for the causal kernel's pairs)."""
    w = workloads.ATTN_WORKLOADS[name]
    q, k, v = (x.to(dev) for x in workloads.make_attention_inputs(w))
    out = q.new_empty(q.shape)

    def launch():
        tg.attention(q, k, v, causal=w.causal, scale=w.scale, out=out)

    wall, ev, _ = bench.time_launches(launch, steps, 5, stream, warm_s=1.0)
    # the launch's grid: 128 queries per workgroup (256 for the non-causal
    # kernel at head dim 64); the causal kernel pairs query blocks
    bm = 256 if w.D == 64 and not w.causal else 128
    q_blocks = (w.N + bm - 1) // bm
    groups = w.B * w.H * ((q_blocks + 1) // 2 if w.causal else q_blocks)
    buf = (ctypes.c_ulonglong * (8 * groups))()
    reader = getattr(lib, READER["attention_fwd_kernel"])
    reader.restype = ctypes.c_int
    reader.argtypes = [ctypes.c_void_p, ctypes.c_int]
    if reader(ctypes.addressof(buf), groups) != 0:
        raise RuntimeError("reading the stamps failed")
    stamps = np.frombuffer(buf, dtype=np.uint64).reshape(groups, 8)
    print(f"{name}: {w.description}", flush=True)
    print(f"  kernel attention_fwd_kernel; {steps}-launch graph: {ev * 1e3:.3f} us per launch (HIP events)", flush=True)
    for line in summarize(stamps, PHASES["attention_fwd_kernel"]):
        print(line, flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("workloads", nargs="*")
    ap.add_argument("--build", action="store_true", help="build the profiling library and exit")
    ap.add_argument("--config", type=int, default=-1, help="force a tile configuration id")
    ap.add_argument("--steps", type=int, default=200)
    args = ap.parse_args()
    if args.build:
        build_profiling_library()
        return 0

    sys.path.insert(0, ROOT)
    import torch

    import bench
    import dense_gemm_epilogues_tiled_amd as tg
    import workloads

    if not os.path.exists(LIB):
        raise SystemExit(f"{LIB} is missing: run python -m dense_gemm_epilogues_tiled_amd.phases --build")
    tg.LIB_PATH = LIB
    lib = tg.load(build_if_missing=False)
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    for name in args.workloads:
        if name in workloads.ATTN_WORKLOADS:
            attention_phases(name, lib, dev, stream, args.steps, bench, tg, workloads)
            continue
        w = workloads.WORKLOADS[name]
        A, B, bias = workloads.make_inputs(w)
        Ad, Bd = A.to(dev), B.to(dev)
        bd = bias.to(dev) if bias is not None else None
        C = torch.empty((w.M, w.N), dtype=torch.float32 if w.epilogue == "softmax" else Ad.dtype, device=dev)
        cfg = (tg.configs()[args.config] if args.config >= 0 else
               tg.query_config(w.M, w.N, w.K, Ad.dtype, w.epilogue, w.b_col_major))
        kernel = bench.kernel_name(cfg)
        if kernel not in PHASES:
            print(f"{name}: kernel {kernel} is not instrumented", flush=True)
            continue

        def launch():
            tg.gemm(Ad, Bd, bd, epilogue=w.epilogue, b_col_major=w.b_col_major, alpha=w.alpha, out=C,
                    config_id=args.config)

        wall, ev, _ = bench.time_launches(launch, args.steps, 10, stream, warm_s=1.0)
        groups = (w.M + cfg["bm"] - 1) // cfg["bm"] * (1 if cfg["kind"] == 1 else (w.N + cfg["bn"] - 1) // cfg["bn"])
        buf = (ctypes.c_ulonglong * (8 * groups))()
        reader = getattr(lib, READER[kernel])
        reader.restype = ctypes.c_int
        reader.argtypes = [ctypes.c_void_p, ctypes.c_int]
        rc = reader(ctypes.addressof(buf), groups)
        if rc != 0:
            raise RuntimeError(f"reading the stamps failed ({rc})")
        stamps = np.frombuffer(buf, dtype=np.uint64).reshape(groups, 8)
        print(f"{name}: {w.description}", flush=True)
        print(f"  kernel {kernel}, configuration {cfg['id']} ({cfg['bm']}x{cfg['bn']}x{cfg['bk']}, "
              f"{cfg['waves']} waves); {args.steps}-launch graph: {ev * 1e3:.3f} us per launch (HIP events)")
        for line in summarize(stamps, PHASES[kernel]):
            print(line, flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
