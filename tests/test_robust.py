"""GPU robustness: writes stay inside C, results are bitwise repeatable,
and a seeded sweep of odd shapes matches the oracle."""

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
GUARD = 4096  # elements of canary on each side of C


def _guarded_out(M, N, dtype):
    """C carved out of a larger buffer whose margins hold a canary pattern."""
    buf = torch.full((GUARD + M * N + GUARD,), -12345.0 if dtype != torch.float32 else -7.0, dtype=dtype,
                     device=DEV)
    return buf, buf[GUARD:GUARD + M * N].view(M, N)


@pytest.mark.parametrize("cfg", GEMM_IDS)
def test_no_writes_outside_c(cfg):
    c = tg.configs()[cfg]
    M, N, K = c["bm"] + 3, c["bn"] + 8, 64
    A = workloads.random_matrix((M, K), 5, "bf16").to(DEV)
    B = workloads.random_matrix((K, N), 6, "bf16").to(DEV)
    bias = workloads.random_matrix((N,), 7, "bf16").to(DEV)
    buf, C = _guarded_out(M, N, torch.bfloat16)
    before = buf.clone()
    tg.gemm(A, B, bias, epilogue="relu", out=C, config_id=cfg)
    torch.cuda.synchronize()
    assert torch.equal(buf[:GUARD], before[:GUARD])
    assert torch.equal(buf[GUARD + M * N:], before[GUARD + M * N:])
    assert not torch.any(C == -12345.0)


def test_softmax_no_writes_outside_c():
    M, N, K = 21, 1000, 72
    A = workloads.random_matrix((M, K), 8, "f16").to(DEV)
    B = workloads.random_matrix((N, K), 9, "f16").to(DEV)
    buf, C = _guarded_out(M, N, torch.float32)
    before = buf.clone()
    tg.gemm(A, B, epilogue="softmax", b_col_major=True, alpha=0.125, out=C)
    torch.cuda.synchronize()
    assert torch.equal(buf[:GUARD], before[:GUARD])
    assert torch.equal(buf[GUARD + M * N:], before[GUARD + M * N:])


@pytest.mark.parametrize("name", ["C3", "C4b", "C5"])
def test_bitwise_repeatable(name):
    """A fixed reduction order: 20 launches give identical bits (a missing LDS
    barrier or wait would show up as run-to-run differences)."""
    w = workloads.WORKLOADS[name]
    A, B, bias = workloads.make_inputs(w)
    Ad, Bd = A.to(DEV), B.to(DEV)
    bd = bias.to(DEV) if bias is not None else None
    first = tg.gemm(Ad, Bd, bd, epilogue=w.epilogue, b_col_major=w.b_col_major, alpha=w.alpha)
    for _ in range(19):
        again = tg.gemm(Ad, Bd, bd, epilogue=w.epilogue, b_col_major=w.b_col_major, alpha=w.alpha)
        assert torch.equal(again, first)
    torch.cuda.synchronize()


def test_random_shape_sweep():
    rng = np.random.default_rng(2024)
    for i in range(24):
        M = int(rng.integers(1, 700))
        N = 8 * int(rng.integers(1, 90))
        K = 8 * int(rng.integers(0, 60))
        dtype = ["f16", "bf16"][i % 2]
        bcol = bool(rng.integers(0, 2))
        epi = ["none", "bias", "relu", "gelu", "softmax"][i % 5]
        print(f"[robust] sweep {i}: {M}x{N}x{K} {dtype} bcol={bcol} {epi}", flush=True)
        A = workloads.random_matrix((M, K), 300 + i, dtype, scale=0.3)
        B = workloads.random_matrix((N, K) if bcol else (K, N), 400 + i, dtype, scale=0.3)
        bias = workloads.random_matrix((N,), 500 + i, dtype) if epi in ("bias", "relu", "gelu") else None
        Cd = tg.gemm(A.to(DEV), B.to(DEV), bias.to(DEV) if bias is not None else None, epilogue=epi,
                     b_col_major=bcol, alpha=0.5)
        torch.cuda.synchronize()
        y = oracle.gemm(A, B, bias, M, N, K, dtype, epi, b_col_major=bcol, alpha=0.5)
        assert_accept(to_f64(Cd), y, "f32" if epi == "softmax" else dtype, f"sweep {i}", small=True)
