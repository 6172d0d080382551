"""GPU: the run-time autotuner.  For each problem the search must find valid
candidates, leave the winner's result in C (checked against the oracle),
cache the winner so that tg_gemm and the query use it (checked against the
oracle again), and survive a save / clear / load round trip."""

import pytest
import torch

import oracle
import workloads
from _compare import assert_accept, to_f64

tg = pytest.importorskip("dense_gemm_epilogues_tiled_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _clean_cache():
    tg.tg_autotune_cache_clear()
    yield
    tg.tg_autotune_cache_clear()


CASES = [
    # M, N, K, dtype, epilogue, b_col_major, alpha
    (2048, 2048, 2048, "f16", "gelu", False, 1.0),
    (1000, 600, 72, "bf16", "relu", True, 0.5),
    (333, 1024, 128, "f16", "softmax", True, 0.125),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}-{c[3]}-{c[4]}")
def test_autotune_finds_caches_and_matches_oracle(case, tmp_path):
    M, N, K, dt, epi, bcol, alpha = case
    print(f"[autotune] {case}", flush=True)
    A = workloads.random_matrix((M, K), 1100 + M, dt, "normal", K ** -0.5)
    B = workloads.random_matrix((N, K) if bcol else (K, N), 1200 + N, dt, "normal", K ** -0.5)
    bias = workloads.random_matrix((N,), 1300, dt) if epi in ("bias", "relu", "gelu") else None
    out_dt = "f32" if epi == "softmax" else dt
    y = oracle.gemm(A, B, bias, M, N, K, dt, epi, b_col_major=bcol, alpha=alpha)
    Ad, Bd = A.to(DEV), B.to(DEV)
    bd = bias.to(DEV) if bias is not None else None

    r = tg.autotune(Ad, Bd, bd, epilogue=epi, b_col_major=bcol, alpha=alpha, iters=3)
    torch.cuda.synchronize()
    print(f"[autotune] best {r['config']['id']} gm={r['config']['group_m']} x={r['config']['xcd_remap']} "
          f"{r['us']:.2f} us, {r['valid']}/{r['candidates']} valid", flush=True)
    assert r["valid"] >= 1 and r["candidates"] >= r["valid"] and r["us"] > 0
    assert (r["M"], r["N"], r["K"], r["b_col_major"]) == (M, N, K, int(bcol))
    assert_accept(to_f64(r["out"]), y, out_dt, "autotune output")

    # the cache now drives the lookup and the plain call
    q = tg.query_config(M, N, K, Ad.dtype, epi, bcol)
    assert (q["id"], q["group_m"], q["xcd_remap"]) == (r["config"]["id"], r["config"]["group_m"],
                                                       r["config"]["xcd_remap"])
    C = tg.gemm(Ad, Bd, bd, epilogue=epi, b_col_major=bcol, alpha=alpha)
    torch.cuda.synchronize()
    assert_accept(to_f64(C), y, out_dt, "gemm after autotune")

    # persistence
    p = str(tmp_path / "cache.txt")
    assert tg.tg_autotune_cache_save(p) == tg.TG_OK
    tg.tg_autotune_cache_clear()
    assert tg.tg_autotune_cache_load(p) == (tg.TG_OK, 1, 0)
    q2 = tg.query_config(M, N, K, Ad.dtype, epi, bcol)
    assert (q2["id"], q2["group_m"], q2["xcd_remap"]) == (q["id"], q["group_m"], q["xcd_remap"])
