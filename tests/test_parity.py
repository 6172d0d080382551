"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

The five workloads at their full sizes and in the launch configuration the
benchmark times (the library's own table lookup), compared element by
element (the 8192^3 case on 65,536 seeded positions), then ragged shapes
across the tile edges of every compiled variant, both B layouts, both dtypes
and every epilogue, K = 0 and empty outputs.
"""

import itertools

import numpy as np
import pytest
import torch

import oracle
import workloads
from _compare import assert_accept, to_f64

tg = pytest.importorskip("dense_gemm_epilogues_tiled_amd")

pytestmark = pytest.mark.gpu
GEMM_IDS = [c["id"] for c in tg.configs() if c["kind"] == tg.TG_KERNEL_GEMM]

DEV = "cuda:0"


def _run(A, B, bias, w_epi, b_col_major=False, alpha=1.0, config_id=-1):
    Ad, Bd = A.to(DEV), B.to(DEV)
    bd = bias.to(DEV) if bias is not None else None
    C = tg.gemm(Ad, Bd, bd, epilogue=w_epi, b_col_major=b_col_major, alpha=alpha, config_id=config_id)
    torch.cuda.synchronize()
    return C


def _oracle_dtype(t):
    return "f16" if t.dtype == torch.float16 else "bf16"


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4b", "C5"])
def test_workload_full(name):
    w = workloads.WORKLOADS[name]
    print(f"[parity] {name}: {w.description}", flush=True)
    A, B, bias = workloads.make_inputs(w)
    C = _run(A, B, bias, w.epilogue, w.b_col_major, w.alpha)
    y = oracle.gemm(A, B, bias, w.M, w.N, w.K, w.dtype, w.epilogue, b_col_major=w.b_col_major, alpha=w.alpha)
    s = assert_accept(to_f64(C), y, w.out_dtype, name)
    print(f"[parity] {name}: {s}", flush=True)


def test_workload_8192_sampled():
    w = workloads.WORKLOADS["C4a"]
    print(f"[parity] C4a: {w.description}", flush=True)
    A, B, bias = workloads.make_inputs(w)
    C = _run(A, B, bias, w.epilogue)
    rows, cols = workloads.sample_positions(w.M, w.N, w.sample, w.seeds[3])
    y = oracle.gemm_sampled(A, B, bias, rows, cols, w.M, w.N, w.K, w.dtype, w.epilogue)
    g = to_f64(C[torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)])
    s = assert_accept(g, y, w.out_dtype, "C4a sampled")
    print(f"[parity] C4a: {s}", flush=True)


def _gemm_variants():
    return [c["id"] for c in tg.configs() if c["kind"] == tg.TG_KERNEL_GEMM]


def _softmax_variants():
    return [c for c in tg.configs() if c["kind"] == tg.TG_KERNEL_GEMM_SOFTMAX]


@pytest.mark.parametrize("cfg", GEMM_IDS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("b_col_major", [False, True])
def test_ragged_shapes_every_variant(cfg, dtype, b_col_major):
    """M, N, K straddling tile edges (M, N: tile +- one row / one 8-column group; K: one K step +- 8)."""
    c = tg.configs()[cfg]
    bm, bn = c["bm"], c["bn"]
    shapes = [(bm + 1, bn + 8, 72), (2 * bm - 1, bn - 8, 56), (3, 8, 8), (bm, 2 * bn, 136)]
    for i, (M, N, K) in enumerate(shapes):
        print(f"[parity] cfg={cfg} {dtype} bcol={b_col_major} M={M} N={N} K={K}", flush=True)
        seed = 1000 + 10 * cfg + i
        A = workloads.random_matrix((M, K), seed, dtype, scale=0.25)
        B = workloads.random_matrix((N, K) if b_col_major else (K, N), seed + 1, dtype, scale=0.25)
        bias = workloads.random_matrix((N,), seed + 2, dtype)
        for epi in ("none", "bias", "relu", "gelu"):
            bb = bias if epi != "none" else None
            C = _run(A, B, bb, epi, b_col_major, alpha=0.75, config_id=cfg)
            y = oracle.gemm(A, B, bb, M, N, K, dtype, epi, b_col_major=b_col_major, alpha=0.75)
            assert_accept(to_f64(C), y, dtype, f"cfg{cfg} {dtype} {epi} {M}x{N}x{K}", small=True)


@pytest.mark.parametrize("cfg", GEMM_IDS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("b_col_major", [False, True])
def test_long_k_every_variant(cfg, dtype, b_col_major):
    """K = 1000: 16 K steps of 64 (32 of 32), so every variant's LDS ring wraps
    several times, plus a 40-deep K tail; edge tiles in M and N."""
    c = tg.configs()[cfg]
    M, N, K = c["bm"] + 16, c["bn"] + 8, 1000
    print(f"[parity] long K cfg={cfg} {dtype} bcol={b_col_major} M={M} N={N} K={K}", flush=True)
    seed = 3000 + 10 * cfg
    A = workloads.random_matrix((M, K), seed, dtype, scale=1 / 32)
    B = workloads.random_matrix((N, K) if b_col_major else (K, N), seed + 1, dtype, scale=1 / 32)
    bias = workloads.random_matrix((N,), seed + 2, dtype)
    for epi in ("none", "gelu"):
        bb = bias if epi != "none" else None
        C = _run(A, B, bb, epi, b_col_major, config_id=cfg)
        y = oracle.gemm(A, B, bb, M, N, K, dtype, epi, b_col_major=b_col_major)
        assert_accept(to_f64(C), y, dtype, f"cfg{cfg} {dtype} {epi} {M}x{N}x{K}", small=True)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("b_col_major", [True, False])
def test_softmax_shapes_every_variant(dtype, b_col_major):
    for c in _softmax_variants():
        if c["b_col_major"] >= 0 and c["b_col_major"] != int(b_col_major):
            continue  # variant built for the other B layout
        for (M, N, K) in [(17, 8, 8), (33, 1000, 72), (16, c["bn"], 128), (5, c["bn"] - 8, 40), (20, 64, 0),
                          (70, c["bn"], 200)]:
            print(f"[parity] softmax cfg={c['id']} {dtype} bcol={b_col_major} M={M} N={N} K={K}", flush=True)
            seed = 7000 + M + N + K
            A = workloads.random_matrix((M, K), seed, dtype)
            B = workloads.random_matrix((N, K) if b_col_major else (K, N), seed + 1, dtype)
            alpha = float(np.float32(1 / np.sqrt(max(K, 1))))
            C = _run(A, B, None, "softmax", b_col_major, alpha=alpha, config_id=c["id"])
            y = oracle.gemm(A, B, None, M, N, K, dtype, "softmax", b_col_major=b_col_major, alpha=alpha)
            assert_accept(to_f64(C), y, "f32", f"softmax cfg{c['id']} {M}x{N}x{K}", small=True)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_k_zero_gives_epilogue_of_bias(dtype):
    M, N = 37, 24
    bias = workloads.random_matrix((N,), 55, dtype)
    A = torch.zeros((M, 0), dtype=workloads.TORCH_DTYPES[dtype])
    B = torch.zeros((0, N), dtype=workloads.TORCH_DTYPES[dtype])
    for epi in ("bias", "relu", "gelu"):
        C = _run(A, B, bias, epi)
        y = oracle.gemm(A, B, bias, M, N, 0, dtype, epi)
        assert_accept(to_f64(C), y, dtype, f"K=0 {epi}", small=True)
    C = _run(A, B, None, "softmax")
    np.testing.assert_allclose(to_f64(C), np.full((M, N), 1.0 / N), rtol=1e-6)


@pytest.mark.parametrize("cfg", GEMM_IDS)
def test_k_zero_every_variant(cfg):
    """K = 0 through each compiled GEMM variant: C = epilogue(bias) (no K step runs)."""
    M, N = 37, 24
    bias = workloads.random_matrix((N,), 56, "f16")
    A = torch.zeros((M, 0), dtype=torch.float16)
    B = torch.zeros((0, N), dtype=torch.float16)
    for epi in ("none", "bias", "gelu"):
        bb = bias if epi != "none" else None
        C = _run(A, B, bb, epi, config_id=cfg)
        y = oracle.gemm(A, B, bb, M, N, 0, "f16", epi)
        assert_accept(to_f64(C), y, "f16", f"cfg{cfg} K=0 {epi}", small=True)


def test_empty_outputs():
    for (M, N, K) in [(0, 64, 64), (64, 0, 64), (0, 0, 0)]:
        A = torch.zeros((M, K), dtype=torch.float16, device=DEV)
        B = torch.zeros((K, N), dtype=torch.float16, device=DEV)
        C = tg.gemm(A, B)
        assert C.shape == (M, N)
    torch.cuda.synchronize()


def test_tg_gemm_plain_entry_point():
    """tg_gemm (alpha = 1, row-major B) through the raw C signature."""
    w = workloads.WORKLOADS["C1"]
    A, B, _ = workloads.make_inputs(w)
    Ad, Bd = A.to(DEV), B.to(DEV)
    C = torch.empty((w.M, w.N), dtype=torch.float16, device=DEV)
    rc = tg.tg_gemm(Ad.data_ptr(), Bd.data_ptr(), None, C.data_ptr(), w.M, w.N, w.K, tg.TG_DTYPE_F16,
                    tg.TG_EPI_NONE, torch.cuda.current_stream().cuda_stream)
    assert rc == tg.TG_OK
    torch.cuda.synchronize()
    y = oracle.gemm(A, B, None, w.M, w.N, w.K, "f16", "none")
    assert_accept(to_f64(C), y, "f16", "tg_gemm C1")


def test_nondefault_stream():
    w = workloads.WORKLOADS["C1"]
    A, B, _ = workloads.make_inputs(w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        C = tg.gemm(A.to(DEV), B.to(DEV))
    s.synchronize()
    y = oracle.gemm(A, B, None, w.M, w.N, w.K, "f16", "none")
    assert_accept(to_f64(C), y, "f16", "side stream")
