"""Launch one GEMM shape repeatedly, for profilers.

    rocprofv3 --pmc <counters> -- python3 -m dense_gemm_epilogues_tiled_amd.profile_run \\
        --shape 2048,2048,64 --dtype f16 --epilogue gelu [--b-col-major] [--config ID] [--launches 10]

Seeded N(0,1)/sqrt(K) operands (bias N(0,1) for the bias epilogues), the
library's own configuration choice unless --config forces one; `--launches`
eager launches after 3 untimed ones.  Prints the configuration and the mean
HIP-event time per launch.  Used to attribute counters to parts of a kernel,
e.g. a scan over K separates per-step costs from per-tile ones.
"""

from __future__ import annotations

import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--shape", required=True, help="M,N,K")
    ap.add_argument("--dtype", default="f16", choices=["f16", "bf16"])
    ap.add_argument("--epilogue", default="none", choices=["none", "bias", "relu", "gelu", "softmax"])
    ap.add_argument("--b-col-major", action="store_true")
    ap.add_argument("--config", type=int, default=-1)
    ap.add_argument("--launches", type=int, default=10)
    args = ap.parse_args()
    M, N, K = (int(v) for v in args.shape.split(","))

    sys.path.insert(0, ROOT)
    import torch

    import dense_gemm_epilogues_tiled_amd as tg
    import workloads

    tg.load(build_if_missing=False)
    dev = torch.device("cuda:0")
    scale = float(K) ** -0.5 if K > 0 else 1.0
    A = workloads.random_matrix((M, K), 1, args.dtype, scale=scale).to(dev)
    B = workloads.random_matrix((N, K) if args.b_col_major else (K, N), 2, args.dtype, scale=scale).to(dev)
    bias = (workloads.random_matrix((N,), 3, args.dtype).to(dev) if args.epilogue in ("bias", "relu", "gelu")
            else None)
    out = torch.empty((M, N), dtype=torch.float32 if args.epilogue == "softmax" else A.dtype, device=dev)

    def launch():
        tg.gemm(A, B, bias, epilogue=args.epilogue, b_col_major=args.b_col_major, out=out, config_id=args.config)

    for _ in range(3):
        launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.launches):
        launch()
    e1.record()
    torch.cuda.synchronize()
    cfg = (tg.configs()[args.config] if args.config >= 0 else
           tg.query_config(M, N, K, A.dtype, args.epilogue, args.b_col_major))
    print(json.dumps({"shape": [M, N, K], "dtype": args.dtype, "epilogue": args.epilogue, "config": cfg["id"],
                      "us_per_launch": round(e0.elapsed_time(e1) * 1e3 / max(args.launches, 1), 3)}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
