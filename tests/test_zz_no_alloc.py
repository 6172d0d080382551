"""GPU: tg_gemm_autotune_noalloc (the autotuner with the library's own fixed
scratch array as its workspace) against tg_gemm_autotune with a caller
workspace, through the C ABI, on two calls in a row, the second with a
smaller problem: the same candidates run, the output of each call matches
the fp64 oracle and the other entry point's output to the parity bar; a
problem whose workspace exceeds the array is refused before any launch."""

import ctypes

import pytest
import torch

import oracle
import workloads
from _compare import TOL, assert_accept, to_f64

tg = pytest.importorskip("dense_gemm_epilogues_tiled_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _args(A, B, bias, C, M, N, K, dtype, epi):
    return tg.tg_gemm_args(A.data_ptr(), B.data_ptr(), bias.data_ptr() if bias is not None else None, C.data_ptr(),
                           M, N, K, dtype, epi, 0, 1.0, -1, 0, -1)


@pytest.mark.parametrize("order", ["noalloc_first", "workspace_first"])
def test_noalloc_matches_workspace_entry_point(order):
    tg.load(build_if_missing=False)
    stream = torch.cuda.current_stream().cuda_stream
    cases = [("f16", "gelu", 520, 392, 264), ("bf16", "relu", 200, 136, 72)]  # second call smaller
    try:
        for i, (dtype, epi, M, N, K) in enumerate(cases):
            print(f"[no-alloc] {order} call {i}: {dtype} {epi} M={M} N={N} K={K}", flush=True)
            A = workloads.random_matrix((M, K), 60 + i, dtype, scale=0.25)
            B = workloads.random_matrix((K, N), 70 + i, dtype, scale=0.25)
            bias = workloads.random_matrix((N,), 80 + i, dtype)
            Ad, Bd, bd = A.to(DEV), B.to(DEV), bias.to(DEV)
            td = workloads.TORCH_DTYPES[dtype]
            code, epi_code = tg.DTYPES[td], tg.EPILOGUES[epi]
            C_na = torch.full((M, N), float("nan"), dtype=td, device=DEV)
            C_ws = torch.full((M, N), float("nan"), dtype=td, device=DEV)

            def run_noalloc():
                rc, e = tg.tg_gemm_autotune_noalloc(_args(Ad, Bd, bd, C_na, M, N, K, code, epi_code), 3, stream)
                assert rc == tg.TG_OK, tg.tg_status_string(rc)
                return e

            def run_workspace():
                rc, need = tg.tg_gemm_autotune_workspace_size(M, N, epi_code)
                assert rc == tg.TG_OK
                ws = torch.empty(need + 256, dtype=torch.uint8, device=DEV)
                base = (ws.data_ptr() + 255) // 256 * 256
                rc, e = tg.tg_gemm_autotune(_args(Ad, Bd, bd, C_ws, M, N, K, code, epi_code), base, need, 3, stream)
                assert rc == tg.TG_OK, tg.tg_status_string(rc)
                torch.cuda.synchronize()
                del ws
                return e

            if order == "noalloc_first":
                e_na, e_ws = run_noalloc(), run_workspace()
            else:
                e_ws, e_na = run_workspace(), run_noalloc()
            torch.cuda.synchronize()
            assert e_na.candidates == e_ws.candidates and e_na.valid >= 1 and e_ws.valid >= 1
            assert e_na.us > 0 and e_ws.us > 0
            y = oracle.gemm(A, B, bias, M, N, K, dtype, epi)
            s_na = assert_accept(to_f64(C_na), y, dtype, f"noalloc {dtype} {epi}")
            assert_accept(to_f64(C_ws), y, dtype, f"workspace {dtype} {epi}")
            # the two entry points' outputs against each other, at the per-element bar
            g, r = to_f64(C_na), to_f64(C_ws)
            atol, rtol = TOL[dtype]
            assert (abs(g - r) <= atol + rtol * abs(r)).all()
            print(f"[no-alloc] call {i}: winner cfg {e_na.config.id} ({e_na.us:.2f} us) / cfg {e_ws.config.id} "
                  f"({e_ws.us:.2f} us), {e_na.candidates} candidates, {s_na}", flush=True)
    finally:
        tg.tg_autotune_cache_clear()


def test_noalloc_refuses_a_workspace_beyond_the_array():
    tg.load(build_if_missing=False)
    M = N = 8192  # a 128 MiB bf16 output: its workspace exceeds TG_AUTOTUNE_NOALLOC_MAX_BYTES
    rc, need = tg.tg_gemm_autotune_workspace_size(M, N, tg.TG_EPI_NONE)
    assert rc == tg.TG_OK and need > tg.TG_AUTOTUNE_NOALLOC_MAX_BYTES
    x = torch.zeros(16, dtype=torch.bfloat16, device=DEV)  # never touched: the size check comes first
    args = tg.tg_gemm_args(x.data_ptr(), x.data_ptr(), None, x.data_ptr(), M, N, 64, tg.TG_DTYPE_BF16,
                           tg.TG_EPI_NONE, 0, 1.0, -1, 0, -1)
    rc, _ = tg.tg_gemm_autotune_noalloc(args, 3, torch.cuda.current_stream().cuda_stream)
    assert rc == tg.TG_ERR_UNSUPPORTED
    rc, _ = tg.tg_gemm_autotune_noalloc(None, 3, None)
    assert rc == tg.TG_ERR_INVALID_ARG
