"""GPU parity at the largest sizes the ABI accepts along K (2^20) and N (2^24),
and for the attention forward at its longest sequence (2^20).

These are where the kernels' 32-bit byte offsets inside a tile come closest
to their limit: one 64-deep step of a row-major B at N = 2^24 spans 2^31
bytes, and a 256-row A tile at K = 2^20 spans 2^29.  Every GEMM variant runs
each case; the row softmax runs the K limit.

At N = 2^24, B and bias repeat a seeded 4096-column block (B[:, n] =
B0[:, n mod 4096], bias[n] = bias0[n mod 4096]), so the exact result repeats
too: the oracle computes the M x 4096 block once, and the GPU output is
compared with it on sampled columns spread over the whole row, the first and
the last tile included.
"""

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
K_MAX = 1 << 20
N_MAX = 1 << 24
PERIOD = 4096


@pytest.fixture(scope="module")
def k_limit_case():
    M, N, K = 64, 64, K_MAX
    A = workloads.random_matrix((M, K), 9101, "f16", scale=K ** -0.5)
    B = workloads.random_matrix((K, N), 9102, "f16", scale=K ** -0.5)
    bias = workloads.random_matrix((N,), 9103, "f16")
    y = oracle.gemm(A, B, bias, M, N, K, "f16", "gelu")
    return M, N, K, A.to(DEV), B.to(DEV), bias.to(DEV), y


@pytest.mark.parametrize("cfg", GEMM_IDS)
def test_k_at_limit_every_variant(k_limit_case, cfg):
    M, N, K, Ad, Bd, bd, y = k_limit_case
    print(f"[max] K={K} cfg={cfg} f16 gelu M={M} N={N}", flush=True)
    C = tg.gemm(Ad, Bd, bd, epilogue="gelu", config_id=cfg)
    assert_accept(to_f64(C), y, "f16", f"K = 2^20 cfg{cfg}")


def test_k_at_limit_softmax():
    M, N, K = 16, 64, K_MAX
    A = workloads.random_matrix((M, K), 9111, "f16")
    B = workloads.random_matrix((N, K), 9112, "f16")
    alpha = float(np.float32(K ** -0.5))
    y = oracle.gemm(A, B, None, M, N, K, "f16", "softmax", b_col_major=True, alpha=alpha)
    Ad, Bd = A.to(DEV), B.to(DEV)
    for c in tg.configs():
        if c["kind"] != tg.TG_KERNEL_GEMM_SOFTMAX or c["b_col_major"] == 0:
            continue
        print(f"[max] softmax K={K} cfg={c['id']}", flush=True)
        C = tg.gemm(Ad, Bd, None, epilogue="softmax", b_col_major=True, alpha=alpha, config_id=c["id"])
        assert_accept(to_f64(C), y, "f32", f"softmax K = 2^20 cfg{c['id']}")


@pytest.fixture(scope="module", params=[False, True], ids=["B_row_major", "B_col_major"])
def n_limit_case(request):
    b_col_major = request.param
    M, N, K = 20, N_MAX, 64
    A = workloads.random_matrix((M, K), 9121, "bf16", scale=K ** -0.5)
    B0 = workloads.random_matrix((PERIOD, K) if b_col_major else (K, PERIOD), 9122, "bf16", scale=K ** -0.5)
    bias0 = workloads.random_matrix((PERIOD,), 9123, "bf16")
    y0 = oracle.gemm(A, B0, bias0, M, PERIOD, K, "bf16", "relu", b_col_major=b_col_major)
    reps = N // PERIOD
    B0d = B0.to(DEV)
    Bd = B0d.repeat(reps, 1) if b_col_major else B0d.repeat(1, reps)
    bd = bias0.to(DEV).repeat(reps)
    rng = np.random.default_rng(9124)
    cols = np.concatenate([np.arange(512), np.arange(N - 512, N), rng.integers(0, N, 3072)])
    yield M, N, K, b_col_major, A.to(DEV), Bd, bd, y0, cols
    del Bd, bd
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg", GEMM_IDS)
def test_n_at_limit_every_variant(n_limit_case, cfg):
    M, N, K, b_col_major, Ad, Bd, bd, y0, cols = n_limit_case
    print(f"[max] N={N} cfg={cfg} bf16 relu M={M} K={K} bcol={b_col_major}", flush=True)
    C = tg.gemm(Ad, Bd, bd, epilogue="relu", b_col_major=b_col_major, config_id=cfg)
    g = to_f64(C[:, torch.from_numpy(cols).to(DEV)])
    assert_accept(g, y0[:, cols % PERIOD], "bf16", f"N = 2^24 cfg{cfg} bcol={b_col_major}")
    del C


@pytest.mark.parametrize("causal", [False, True], ids=["non_causal", "causal"])
@pytest.mark.parametrize("D,dtype", [(64, "bf16"), (128, "f16")])
def test_attention_at_longest_sequence(D, dtype, causal):
    """seq_len = 2^20 (TG_ATTN_MAX_SEQ), one head: the longest key loop and the
    largest query-block index; sampled rows, the first and last query included."""
    B, H, N = 1, 1, 1 << 20
    assert N == tg.TG_ATTN_MAX_SEQ
    seed = 9130 + D + int(causal)
    Q = workloads.random_matrix((B, H, N, D), seed, dtype)
    K = workloads.random_matrix((B, H, N, D), seed + 1, dtype)
    V = workloads.random_matrix((B, H, N, D), seed + 2, dtype)
    scale = float(np.float32(D ** -0.5))
    print(f"[max] attention N={N} D={D} {dtype} causal={causal}", flush=True)
    O = tg.attention(Q.to(DEV), K.to(DEV), V.to(DEV), causal=causal, scale=scale)
    rng = np.random.default_rng(seed + 3)
    rows = np.concatenate([[0, 1, N - 2, N - 1], rng.integers(0, N, 12)])
    y = oracle.attention_rows(Q, K, V, rows, B, H, N, D, dtype, causal, scale)
    got = to_f64(O.reshape(-1, D)[torch.from_numpy(rows).to(DEV)])
    # bf16 probabilities feed the P.V product: the bf16 bar is 1.5 x the
    # error of the correctly rounded output, as for the attention workloads
    assert_accept(got, y, dtype, f"attention N = 2^20 D={D} causal={causal}",
                  floor_factor=1.5 if dtype == "bf16" else None)
