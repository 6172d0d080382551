"""Pins for the CPU oracle (no GPU).

The TileLang pages print no worked example and no output values, so every pin
below comes from a definition that does not depend on the oracle's code:
exact rational arithmetic, integer arithmetic, numpy's own fp16 decoder, the
bfloat16 definition as the top half of a binary32, closed forms of structured
products, textbook values of the normal distribution function and the
defining identities of GELU and softmax.  A dropped term, a wrong sign or
index, a transposed operand, a misplaced bias or a tanh-form GELU each fail at
least one test here.
"""

import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# exact decode of the input formats
# --------------------------------------------------------------------------

def test_f16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros survive
    assert math.copysign(1.0, oracle.f16_to_f64(0x8000)) == -1.0


def test_bf16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# --------------------------------------------------------------------------
# the triple loop
# --------------------------------------------------------------------------

def _bits_np(x: np.ndarray, dtype: str) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(workloads.TORCH_DTYPES[dtype])
    return t.view(torch.int16).numpy().view(np.uint16)


def _values(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _col_major(b_bits: np.ndarray, K: int, N: int) -> np.ndarray:
    """Store logical K x N matrix as N x K row-major (column-major K x N)."""
    return np.ascontiguousarray(b_bits.reshape(K, N).T)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("col_major", [False, True])
def test_identity(dtype, col_major):
    rng = np.random.default_rng(1)
    M, K = 37, 24
    A = _bits_np(rng.standard_normal((M, K)), dtype)
    I = _bits_np(np.eye(K), dtype)
    Ib = _col_major(I, K, K) if col_major else I
    y = oracle.gemm(A, Ib, None, M, K, K, dtype, "none", b_col_major=col_major)
    assert np.array_equal(y, _values(A, dtype).reshape(M, K))
    # I . B = B
    B = _bits_np(rng.standard_normal((K, M)), dtype)
    Bb = _col_major(B, K, M) if col_major else B
    y2 = oracle.gemm(I, Bb, None, K, M, K, dtype, "none", b_col_major=col_major)
    assert np.array_equal(y2, _values(B, dtype).reshape(K, M))


@pytest.mark.parametrize("col_major", [False, True])
def test_permutations(col_major):
    rng = np.random.default_rng(2)
    M, N, K = 19, 23, 17
    A = _bits_np(rng.standard_normal((M, K)), "f16")
    pk = rng.permutation(K)
    P = np.zeros((K, K))
    P[np.arange(K), pk] = 1.0  # (A.P)[:, pk[r]] = A[:, r]
    Pb = _bits_np(P, "f16")
    y = oracle.gemm(A, _col_major(Pb, K, K) if col_major else Pb, None, M, K, K, "f16", "none",
                    b_col_major=col_major)
    av = _values(A, "f16").reshape(M, K)
    assert np.array_equal(y[:, pk], av)
    # row permutation of B: (Q . B)[r, :] = B[q[r], :]
    B = _bits_np(rng.standard_normal((K, N)), "f16")
    q = rng.permutation(K)
    Q = np.zeros((K, K))
    Q[np.arange(K), q] = 1.0
    y2 = oracle.gemm(_bits_np(Q, "f16"), _col_major(B, K, N) if col_major else B, None, K, N, K, "f16", "none",
                     b_col_major=col_major)
    assert np.array_equal(y2, _values(B, "f16").reshape(K, N)[q, :])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_rank_one_closed_form(dtype):
    # A = u 1^T, B = 1 v^T  =>  acc_ij = K u_i v_j exactly (K a power of two)
    rng = np.random.default_rng(3)
    M, N, K = 13, 11, 64
    u = _values(_bits_np(rng.uniform(-2, 2, M), dtype), dtype)
    v = _values(_bits_np(rng.uniform(-2, 2, N), dtype), dtype)
    A = _bits_np(np.repeat(u[:, None], K, axis=1), dtype)
    B = _bits_np(np.repeat(v[None, :], K, axis=0), dtype)
    y = oracle.gemm(A, B, None, M, N, K, dtype, "none")
    assert np.array_equal(y, K * np.outer(u, v))


def test_integer_matrices_exact():
    # small integers are exact in fp16; the result must equal integer matmul
    rng = np.random.default_rng(4)
    for (M, N, K) in [(5, 7, 64), (33, 9, 48), (1, 64, 3)]:
        Ai = rng.integers(-16, 17, (M, K))
        Bi = rng.integers(-16, 17, (K, N))
        y = oracle.gemm(_bits_np(Ai, "f16"), _bits_np(Bi, "f16"), None, M, N, K, "f16", "none")
        assert np.array_equal(y, (Ai @ Bi).astype(np.float64))


def _exact(av, bv, K, M, N):
    return [[sum((Fraction(av[i, k]) * Fraction(bv[k, j]) for k in range(K)), Fraction(0)) for j in range(N)]
            for i in range(M)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_brute_force_all_small_shapes(dtype):
    """Every shape in {1..8}^3, both B layouts, against exact rational sums."""
    rng = np.random.default_rng(5)
    for M, N, K in itertools.product(range(1, 9), repeat=3):
        A = _bits_np(rng.uniform(-1, 1, (M, K)), dtype)
        B = _bits_np(rng.uniform(-1, 1, (K, N)), dtype)
        av, bv = _values(A, dtype).reshape(M, K), _values(B, dtype).reshape(K, N)
        ex = _exact(av, bv, K, M, N)
        y = oracle.gemm(A, B, None, M, N, K, dtype, "none")
        yc = oracle.gemm(A, _col_major(B, K, N), None, M, N, K, dtype, "none", b_col_major=True)
        for i in range(M):
            for j in range(N):
                e = float(ex[i][j])
                assert abs(y[i, j] - e) <= 1e-15 * max(1.0, abs(e)), (M, N, K, i, j)
        assert np.array_equal(y, yc)
        np.testing.assert_allclose(y, av @ bv, rtol=1e-14, atol=1e-15)


def test_alpha_and_bias_placement():
    """x = alpha*acc + bias[j]: bias follows the column index, alpha scales acc only."""
    rng = np.random.default_rng(6)
    M, N, K = 6, 9, 5
    A = _bits_np(rng.uniform(-1, 1, (M, K)), "f16")
    B = _bits_np(rng.uniform(-1, 1, (K, N)), "f16")
    bias = _bits_np(rng.uniform(-1, 1, N), "f16")
    av, bv, cv = _values(A, "f16").reshape(M, K), _values(B, "f16").reshape(K, N), _values(bias, "f16")
    alpha = 0.375
    y = oracle.gemm(A, B, bias, M, N, K, "f16", "bias", alpha=alpha)
    ex = _exact(av, bv, K, M, N)
    for i in range(M):
        for j in range(N):
            e = float(Fraction(alpha) * ex[i][j] + Fraction(cv[j]))
            assert abs(y[i, j] - e) <= 1e-15 * max(1.0, abs(e))


def test_k_zero_gives_epilogue_of_bias():
    N = 8
    bias = _bits_np(np.linspace(-3, 3, N), "bf16")
    cv = _values(bias, "bf16")
    for epi in ("bias", "relu", "gelu"):
        y = oracle.gemm(np.zeros(0, np.uint16), np.zeros(0, np.uint16), bias, 3, N, 0, "bf16", epi)
        assert np.array_equal(y, np.tile(oracle.act(cv, epi), (3, 1)))


def test_empty_shapes_are_noops():
    y = oracle.gemm(np.zeros(0, np.uint16), np.zeros(0, np.uint16), None, 0, 5, 0, "f16", "none")
    assert y.shape == (0, 5)
    y = oracle.gemm(np.zeros(0, np.uint16), np.zeros(0, np.uint16), None, 4, 0, 0, "f16", "softmax")
    assert y.shape == (4, 0)


def test_sampled_equals_full_bitwise_at_2048():
    w = workloads.WORKLOADS["C3"]
    A, B, bias = workloads.make_inputs(w)
    full = oracle.gemm(A, B, bias, w.M, w.N, w.K, w.dtype, w.epilogue)
    rows, cols = workloads.sample_positions(w.M, w.N, 4096, 7)
    s = oracle.gemm_sampled(A, B, bias, rows, cols, w.M, w.N, w.K, w.dtype, w.epilogue)
    assert np.array_equal(s, full[rows, cols])


def test_sampled_col_major_matches_full():
    rng = np.random.default_rng(8)
    M, N, K = 40, 24, 72
    A = _bits_np(rng.standard_normal((M, K)), "bf16")
    B = _bits_np(rng.standard_normal((N, K)), "bf16")
    bias = _bits_np(rng.standard_normal(N), "bf16")
    full = oracle.gemm(A, B, bias, M, N, K, "bf16", "relu", b_col_major=True, alpha=0.5)
    rows, cols = workloads.sample_positions(M, N, 300, 9)
    s = oracle.gemm_sampled(A, B, bias, rows, cols, M, N, K, "bf16", "relu", b_col_major=True, alpha=0.5)
    assert np.array_equal(s, full[rows, cols])


def test_bad_arguments_rejected():
    with pytest.raises(ValueError):
        oracle.gemm(np.zeros(4, np.uint16), np.zeros(4, np.uint16), None, 2, 2, 3, "f16", "none")
    with pytest.raises(ValueError):
        oracle.gemm_sampled(np.zeros(4, np.uint16), np.zeros(4, np.uint16), None, [0], [0], 2, 2, 2, "f16",
                            "softmax")
    with pytest.raises(ValueError):
        oracle.gemm_sampled(np.zeros(4, np.uint16), np.zeros(4, np.uint16), None, [2], [0], 2, 2, 2, "f16", "none")


# --------------------------------------------------------------------------
# epilogue functions
# --------------------------------------------------------------------------

def test_relu_values_and_signed_zero():
    x = np.array([-2.5, -1e-300, -0.0, 0.0, 1e-300, 3.0, -np.inf, np.inf])
    y = oracle.act(x, "relu")
    assert np.array_equal(y, np.array([0, 0, 0, 0, 1e-300, 3.0, 0, np.inf]))


def _golden_phi():
    rows = []
    with open(os.path.join(GOLDEN, "normal_cdf_table.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                x, p = line.split()
                rows.append((float(x), float(p)))
    return rows


def test_gelu_textbook_values():
    rows = _golden_phi()
    assert len(rows) >= 9
    x = np.array([r[0] for r in rows])
    expect = x * np.array([r[1] for r in rows])
    got = oracle.act(x, "gelu")
    # 1 + erf(x/sqrt2) cancels for negative x (about 2.5 digits at x = -3): fp64 still
    # keeps better than 1e-13 relative, far below any alternative form's deviation.
    np.testing.assert_allclose(got, expect, rtol=1e-13, atol=1e-300)
    # the tanh approximation is a different function: it must NOT pass this pin
    tanh_form = 0.5 * x * (1 + np.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))
    assert np.max(np.abs(tanh_form - expect)) > 1e-5


def test_gelu_identities():
    assert oracle.act(np.array([0.0]), "gelu")[0] == 0.0
    x = np.linspace(-10, 10, 2001)
    g, gm = oracle.act(x, "gelu"), oracle.act(-x, "gelu")
    # x*Phi(x) - (-x)*Phi(-x) = x*(Phi(x) + Phi(-x)) = x
    np.testing.assert_allclose(g - gm, x, rtol=1e-15, atol=1e-15)
    # large |x|: GELU -> relu
    assert oracle.act(np.array([40.0]), "gelu")[0] == 40.0
    assert oracle.act(np.array([-40.0]), "gelu")[0] == 0.0 or abs(oracle.act(np.array([-40.0]), "gelu")[0]) < 1e-300


def test_gelu_minimum():
    from scipy.optimize import brentq, minimize_scalar
    from scipy.special import ndtr
    # d/dx [x Phi(x)] = Phi(x) + x phi(x) = 0
    x0 = brentq(lambda t: ndtr(t) + t * math.exp(-t * t / 2) / math.sqrt(2 * math.pi), -2, -0.1)
    r = minimize_scalar(lambda t: oracle.act(np.array([t]), "gelu")[0], bounds=(-2, 0), method="bounded",
                        options={"xatol": 1e-10})
    assert abs(r.x - x0) < 1e-6
    assert abs(r.fun - x0 * ndtr(x0)) < 1e-14
    assert abs(r.fun - (-0.169971)) < 1e-6


def _softmax_oracle(x_rows: np.ndarray) -> np.ndarray:
    """Feed an M x N matrix of fp16-exact values through the oracle's softmax:
    acc = x (A = x, B = I)."""
    M, N = x_rows.shape
    A = _bits_np(x_rows, "f16")
    I = _bits_np(np.eye(N), "f16")
    return oracle.gemm(A, I, None, M, N, N, "f16", "softmax")


def test_softmax_rows_sum_to_one_and_order():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((16, 50)) * 4
    y = _softmax_oracle(x)
    np.testing.assert_allclose(y.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    xv = _values(_bits_np(x, "f16"), "f16").reshape(x.shape)
    assert np.array_equal(np.argmax(y, axis=1), np.argmax(xv, axis=1))
    assert np.all(y > 0)


def test_softmax_uniform_and_single_column():
    y = oracle.gemm(np.zeros(4 * 8, np.uint16), np.zeros(8 * 10, np.uint16), None, 4, 10, 8, "f16", "softmax")
    assert np.array_equal(y, np.full((4, 10), 0.1))
    y1 = _softmax_oracle(np.array([[3.5], [-7.0]]))
    assert np.array_equal(y1, np.ones((2, 1)))


def test_softmax_two_columns_logistic():
    x = np.array([[1.0, -0.5], [2.0, 2.0], [-3.25, 4.0], [0.125, 0.0]])
    y = _softmax_oracle(x)
    d = x[:, 0] - x[:, 1]
    s0 = 1 / (1 + np.exp(-d))
    np.testing.assert_allclose(y[:, 0], s0, rtol=1e-15)
    np.testing.assert_allclose(y[:, 1], 1 / (1 + np.exp(d)), rtol=1e-15)


def test_softmax_invariant_to_row_shift_and_uses_alpha():
    """Append a k column carrying c_i with B row of ones: every x_ij of row i gains c_i."""
    rng = np.random.default_rng(11)
    M, N, K = 7, 12, 6
    xa = rng.uniform(-1, 1, (M, K))
    B = rng.uniform(-1, 1, (K, N))
    c = np.round(rng.uniform(-4, 4, M) * 8) / 8
    A1 = _bits_np(np.hstack([xa, np.zeros((M, 1))]), "f16")
    A2 = _bits_np(np.hstack([xa, c[:, None]]), "f16")
    Bx = _bits_np(np.vstack([B, np.ones((1, N))]), "f16")
    y1 = oracle.gemm(A1, Bx, None, M, N, K + 1, "f16", "softmax", alpha=0.7)
    y2 = oracle.gemm(A2, Bx, None, M, N, K + 1, "f16", "softmax", alpha=0.7)
    np.testing.assert_allclose(y1, y2, rtol=1e-13)
    # alpha is applied before the max: softmax(0.7 x) differs from softmax(x)
    y3 = oracle.gemm(A1, Bx, None, M, N, K + 1, "f16", "softmax", alpha=1.0)
    assert np.max(np.abs(y3 - y1)) > 1e-3
    av = _values(A1, "f16").reshape(M, K + 1)
    bv = _values(Bx, "f16").reshape(K + 1, N)
    x = 0.7 * (av @ bv)
    e = np.exp(x - x.max(axis=1, keepdims=True))
    np.testing.assert_allclose(y1, e / e.sum(axis=1, keepdims=True), rtol=1e-13)
