"""GPU parity of the two bandwidth-bound entry points against the CPU oracle.

tg_vector_add is compared bit for bit: the oracle's result is the correctly
rounded sum, and the kernel's fp32-then-round-once sum must be that same value
for every input, subnormals, infinities and overflow included (NaN results
only need to be NaN on both sides: payloads are not specified).

tg_row_softmax is compared per element against the fp64 oracle within the
fp32-output bound |g - y| <= 1e-4 + 1e-4 |y| (and the 2e-3 relative Frobenius
bound), over every register-capacity bucket of the kernel, ragged row counts,
all three input dtypes, negative / zero alpha, large magnitudes and masked
(-inf) entries; the 16384 x 4096 workload on 256 seeded rows.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from _compare import assert_accept

tg = pytest.importorskip("dense_gemm_epilogues_tiled_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TD = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


# ---- vector addition -----------------------------------------------------------

def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.view(torch.int16).numpy().view(np.uint16)


def _is_nan_bits(b: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return ((b & 0x7F800000) == 0x7F800000) & ((b & 0x7FFFFF) != 0)
    if dtype == "f16":
        return ((b & 0x7C00) == 0x7C00) & ((b & 0x3FF) != 0)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)


def _assert_add_exact(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, dtype: str, what: str):
    want = oracle.vector_add(A, B, dtype)
    got = _bits(C).ravel()
    nan_w = _is_nan_bits(want, dtype)
    nan_g = _is_nan_bits(got, dtype)
    assert np.array_equal(nan_w, nan_g), f"{what}: NaN positions differ ({int((nan_w != nan_g).sum())})"
    bad = np.flatnonzero((got != want) & ~nan_w)
    assert bad.size == 0, (f"{what}: {bad.size} of {got.size} sums differ, first at {bad[0]}: "
                           f"a={_bits(A).ravel()[bad[0]]:#x} b={_bits(B).ravel()[bad[0]]:#x} "
                           f"gpu={got[bad[0]]:#x} oracle={want[bad[0]]:#x}")


def _run_add(A, B, in_place=False):
    Ad, Bd = A.to(DEV), B.to(DEV)
    C = tg.vector_add(Ad, Bd, out=Ad if in_place else None)
    torch.cuda.synchronize()
    return C


def test_vector_add_workload_2p22():
    w = workloads.STREAM_WORKLOADS["V1"]
    print(f"[parity] V1: {w.description}", flush=True)
    A, B = workloads.make_stream_inputs(w)
    _assert_add_exact(A, B, _run_add(A, B), w.dtype, "V1")


def test_vector_add_workload_2p28_sampled():
    """The 3 GiB case: 2^26 threads of 16-byte vectors, so the grid's block
    index runs into the millions; 65,536 seeded positions are checked (the
    operation is elementwise, so the oracle sees just those pairs)."""
    w = workloads.STREAM_WORKLOADS["V2"]
    print(f"[parity] V2: {w.description}", flush=True)
    A, B = workloads.make_stream_inputs(w)
    C = _run_add(A, B)
    g = torch.Generator(device="cpu").manual_seed(w.seeds[2])
    idx = torch.randperm(w.n, generator=g)[:65536]
    idx = torch.cat([idx, torch.tensor([0, w.n - 1])])  # first and last element too
    got = C[idx.to(DEV)]
    _assert_add_exact(A[idx], B[idx], got, w.dtype, "V2 sampled")


def _random_patterns(n: int, dtype: str, seed: int) -> torch.Tensor:
    """Uniformly random bit patterns: every finite value class, subnormals,
    infinities and NaNs included."""
    rng = np.random.default_rng(seed)
    if dtype == "f32":
        return torch.from_numpy(rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32).view(np.int32)).view(
            torch.float32)
    return torch.from_numpy(rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16).view(np.int16)).view(
        TD[dtype])


def _near_patterns(n: int, dtype: str, seed: int):
    """Pairs of close magnitudes and opposite signs (cancellation, carries,
    ties after rounding), plus pairs of small multiples of the smallest
    subnormal (exact in fp32, so the conversion below does not round them)."""
    rng = np.random.default_rng(seed)
    span = 14 if dtype == "f16" else 30
    a = rng.standard_normal(n) * np.exp2(rng.integers(-span, span, n))
    b = -a * (1 + rng.standard_normal(n) * np.exp2(-rng.integers(1, 20, n).astype(np.float64)))
    tiny = {"f16": 2.0 ** -24, "bf16": 2.0 ** -133, "f32": 2.0 ** -149}[dtype]
    k = n // 8
    a[:k] = rng.integers(-2000, 2000, k) * tiny
    b[:k] = rng.integers(-2000, 2000, k) * tiny
    return (torch.from_numpy(a).to(torch.float32).to(TD[dtype]),
            torch.from_numpy(b).to(torch.float32).to(TD[dtype]))


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("n", [1, 7, 8, 9, 4093, 100_003, (1 << 21) + 5])
def test_vector_add_every_bit_pattern_class(dtype, n):
    """Random bit patterns at lengths around the 16-byte vector and the
    256-thread block: whole vectors, a partly filled last block and the
    elements past the last whole vector, which go one per thread."""
    print(f"[parity] vector_add {dtype} n={n} random patterns", flush=True)
    A = _random_patterns(n, dtype, 10 + n % 97)
    B = _random_patterns(n, dtype, 20 + n % 89)
    _assert_add_exact(A, B, _run_add(A, B), dtype, f"{dtype} n={n}")


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_vector_add_cancellation_and_subnormals(dtype):
    print(f"[parity] vector_add {dtype} near-cancellation", flush=True)
    A, B = _near_patterns(65_541, dtype, 7)
    _assert_add_exact(A, B, _run_add(A, B), dtype, f"{dtype} near")


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_vector_add_in_place(dtype):
    print(f"[parity] vector_add {dtype} in place", flush=True)
    A = _random_patterns(50_001, dtype, 3)
    B = _random_patterns(50_001, dtype, 4)
    C = _run_add(A, B, in_place=True)
    _assert_add_exact(A, B, C, dtype, f"{dtype} in place")


def test_vector_add_empty():
    z = torch.empty(0, dtype=torch.float32, device=DEV)
    assert tg.vector_add(z, z).numel() == 0


# ---- standalone row softmax ------------------------------------------------------

def _run_softmax(X, alpha=1.0):
    Y = tg.row_softmax(X.to(DEV), alpha=alpha)
    torch.cuda.synchronize()
    return Y.cpu().double().numpy()


def _check_softmax(X, dtype, alpha, what):
    rows, cols = X.shape
    g = _run_softmax(X, alpha)
    y = oracle.softmax(X, rows, cols, dtype, alpha)
    return assert_accept(g, y, "f32", what)


def test_row_softmax_workload_sampled_rows():
    w = workloads.STREAM_WORKLOADS["S1"]
    print(f"[parity] S1: {w.description}", flush=True)
    X, _ = workloads.make_stream_inputs(w)
    g_all = tg.row_softmax(X.to(DEV), alpha=w.alpha)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cpu").manual_seed(w.seeds[2])
    rows = torch.sort(torch.randperm(w.rows, generator=gen)[:256]).values
    rows = torch.cat([rows, torch.tensor([0, w.rows - 1])])
    g = g_all[rows.to(DEV)].cpu().double().numpy()
    Xs = X[rows].contiguous()
    y = oracle.softmax(Xs, Xs.shape[0], w.cols, w.dtype, w.alpha)
    s = assert_accept(g, y, "f32", "S1 sampled rows")
    print(f"[parity] S1: {s}", flush=True)


_COLS = {
    # every register-capacity bucket (64 lanes x 16 bytes x {1, 2, 4, 8, 16}),
    # its edges and a value inside
    "f16": [8, 16, 504, 512, 520, 1024, 1032, 2048, 2056, 4096, 4104, 8192],
    "bf16": [8, 512, 520, 2048, 4104, 8192],
    "f32": [4, 252, 256, 260, 1024, 1028, 2048, 2052, 4096],
}


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_row_softmax_every_bucket(dtype):
    for i, cols in enumerate(_COLS[dtype]):
        for rows in (1, 5, 37):
            print(f"[parity] row_softmax {dtype} rows={rows} cols={cols}", flush=True)
            X = workloads.random_matrix((rows, cols), 900 + 7 * i + rows, dtype, "normal", 2.0)
            _check_softmax(X, dtype, 1.0, f"{dtype} {rows}x{cols}")


@pytest.mark.parametrize("alpha", [-0.75, 0.0, 0.125, 3.0])
def test_row_softmax_alpha(alpha):
    print(f"[parity] row_softmax alpha={alpha}", flush=True)
    X = workloads.random_matrix((33, 1024), 77, "bf16", "normal", 1.0)
    _check_softmax(X, "bf16", alpha, f"alpha={alpha}")


def test_row_softmax_large_magnitudes():
    """Entries up to ~6e4 (fp16's range): without the max subtraction exp
    overflows; with it most entries underflow to exactly 0 and the max gets ~1."""
    print("[parity] row_softmax large magnitudes", flush=True)
    X = workloads.random_matrix((19, 2048), 88, "f16", "uniform", 60000.0)
    _check_softmax(X, "f16", 1.0, "large")
    X = workloads.random_matrix((19, 1000), 89, "f32", "normal", 1e30)
    _check_softmax(X, "f32", 1.0, "huge f32")


def test_row_softmax_masked_entries():
    """-inf entries (a causal mask) get exactly 0; a row that is -inf
    everywhere is NaN on both sides."""
    print("[parity] row_softmax masked", flush=True)
    rows, cols = 64, 512
    X = workloads.random_matrix((rows, cols), 99, "f16", "normal", 1.0)
    mask = torch.arange(cols)[None, :] > torch.arange(rows)[:, None] * (cols // rows)
    X = X.masked_fill(mask, float("-inf"))
    X[rows - 1] = float("-inf")
    g = _run_softmax(X)
    y = oracle.softmax(X, rows, cols, "f16", 1.0)
    assert np.all(np.isnan(g[rows - 1])) and np.all(np.isnan(y[rows - 1]))
    assert np.all(g[:-1][mask[:-1].numpy()] == 0.0)
    assert_accept(g[:-1], y[:-1], "f32", "masked")


def test_row_softmax_empty():
    z = torch.empty((0, 64), dtype=torch.float16, device=DEV)
    assert tg.row_softmax(z).shape == (0, 64)
    z = torch.empty((5, 0), dtype=torch.float32, device=DEV)
    assert tg.row_softmax(z).shape == (5, 0)
