"""Pins for the oracle's vector addition, rounding and standalone row softmax
(no GPU).

Each function is checked against something that does not share its code:
numpy's IEEE binary16 / binary32 conversions and arithmetic, torch's bfloat16
conversion and arithmetic (on inputs where no intermediate rounding can
occur), the midpoints between adjacent representable values (where ties must
go to the even neighbour), closed forms of softmax, and the already pinned
GEMM oracle's softmax epilogue with B = I.  A wrong rounding direction, a lost
tie rule, a mishandled subnormal or overflow, a dropped operand or a wrong
normalisation each fail at least one test here.
"""

import math

import numpy as np
import pytest
import torch

import oracle


def _f16_grid():
    """Every finite fp16 value and every midpoint between adjacent ones."""
    v = np.arange(0, 0x7c00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (v[:-1] + v[1:]) / 2  # exact in fp64
    over = np.array([65504.0, 65519.99, 65520.0, 65536.0, 1e6, math.inf])
    x = np.concatenate([v, mids, over, [2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26]])
    return np.concatenate([x, -x])


# --------------------------------------------------------------------------
# rounding fp64 -> fp16 / bf16 / fp32
# --------------------------------------------------------------------------

def test_round_f16_matches_numpy_on_every_value_and_midpoint():
    x = _f16_grid()
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = oracle.round_to(x, "f16")
    assert np.array_equal(got, ref)


def test_round_f16_random_magnitudes():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(200_000) * np.exp2(rng.uniform(-30, 17, 200_000))
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.round_to(x, "f16"), ref)


def test_round_f32_matches_numpy():
    rng = np.random.default_rng(8)
    x = rng.standard_normal(200_000) * np.exp2(rng.uniform(-160, 130, 200_000))
    f = rng.standard_normal(50_000).astype(np.float32)
    nxt = np.nextafter(f, np.float32(np.inf))
    mids = (f.astype(np.float64) + nxt.astype(np.float64)) / 2  # ties, exact in fp64
    x = np.concatenate([x, mids, [3.4028235677973366e38, 3.40282357e38, 1e39, 2.0 ** -150, 2.0 ** -149, 0.0, -0.0]])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32).view(np.uint32)
    assert np.array_equal(oracle.round_to(x, "f32"), ref)


def test_round_bf16_matches_torch_on_fp32_inputs():
    # fp32 inputs (so a conversion path through fp32 cannot round twice), plus
    # every midpoint between adjacent bf16 values of a range of binades
    rng = np.random.default_rng(9)
    f = (rng.standard_normal(100_000) * np.exp2(rng.uniform(-130, 125, 100_000))).astype(np.float32)
    b = np.arange(0x0000, 0x7f80, 37, dtype=np.uint32) << 16  # bf16 values as fp32 bit patterns
    lo = b.view(np.float32).astype(np.float64)
    hi = ((b + (1 << 16)).view(np.float32)).astype(np.float64)
    mids = ((lo + hi) / 2).astype(np.float32)  # representable in fp32
    x = np.concatenate([f, mids, -mids]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round_to(x.astype(np.float64), "bf16"), ref)


def test_round_ties_go_to_even_by_hand():
    assert list(oracle.round_to([1 + 2 ** -11, 1 + 3 * 2 ** -11], "f16")) == [0x3C00, 0x3C02]
    assert list(oracle.round_to([1 + 2 ** -8, 1 + 3 * 2 ** -8], "bf16")) == [0x3F80, 0x3F82]
    assert list(oracle.round_to([1 + 2 ** -24, 1 + 3 * 2 ** -24], "f32")) == [0x3F800000, 0x3F800002]
    assert list(oracle.round_to([-0.0, 0.0], "f16")) == [0x8000, 0x0000]


def test_f32_decode_matches_bit_reinterpretation():
    rng = np.random.default_rng(10)
    w = rng.integers(0, 2 ** 32, 100_000, dtype=np.uint64).astype(np.uint32)
    w = np.concatenate([w, np.array([0, 0x80000000, 1, 0x7f7fffff, 0x7f800000, 0xff800000], dtype=np.uint32)])
    with np.errstate(invalid="ignore"):
        ref = w.view(np.float32).astype(np.float64)
    got = np.array([oracle.f32_to_f64(int(v)) for v in w])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# --------------------------------------------------------------------------
# vector addition
# --------------------------------------------------------------------------

def _special(dtype):
    big = {"f16": 60000.0, "bf16": 3e38, "f32": 3e38}[dtype]
    tiny = {"f16": 2.0 ** -24, "bf16": 2.0 ** -133, "f32": 2.0 ** -149}[dtype]
    a = [1.0, -1.0, 0.0, -0.0, big, big, tiny, tiny, -tiny, 1.0, 3.0]
    b = [-1.0, 1.0, -0.0, -0.0, big, -big, tiny, -tiny, tiny, 0.0, 2.0 ** -12]
    return np.array(a), np.array(b)


def test_vector_add_f32_matches_ieee():
    rng = np.random.default_rng(11)
    a = (rng.standard_normal(100_000) * np.exp2(rng.uniform(-20, 20, 100_000))).astype(np.float32)
    b = (rng.standard_normal(100_000) * np.exp2(rng.uniform(-20, 20, 100_000))).astype(np.float32)
    sa, sb = _special("f32")
    a = np.concatenate([a, sa.astype(np.float32)])
    b = np.concatenate([b, sb.astype(np.float32)])
    with np.errstate(over="ignore"):
        ref = (a + b).view(np.uint32)
    assert np.array_equal(oracle.vector_add(a, b, "f32"), ref)


def test_vector_add_f16_matches_ieee():
    rng = np.random.default_rng(12)
    a = rng.integers(0, 0x7c00, 100_000).astype(np.uint16) | (rng.integers(0, 2, 100_000).astype(np.uint16) << 15)
    b = rng.integers(0, 0x7c00, 100_000).astype(np.uint16) | (rng.integers(0, 2, 100_000).astype(np.uint16) << 15)
    sa, sb = _special("f16")
    a = np.concatenate([a, sa.astype(np.float16).view(np.uint16)])
    b = np.concatenate([b, sb.astype(np.float16).view(np.uint16)])
    with np.errstate(over="ignore"):
        ref = (a.view(np.float16) + b.view(np.float16)).view(np.uint16)
    assert np.array_equal(oracle.vector_add(a, b, "f16"), ref)


def test_vector_add_bf16_matches_torch():
    g = torch.Generator().manual_seed(13)
    a = (torch.randn(100_000, generator=g) * torch.exp2(torch.rand(100_000, generator=g) * 40 - 20)).to(torch.bfloat16)
    b = (torch.randn(100_000, generator=g) * torch.exp2(torch.rand(100_000, generator=g) * 40 - 20)).to(torch.bfloat16)
    sa, sb = _special("bf16")
    a = torch.cat([a, torch.tensor(sa, dtype=torch.float64).to(torch.bfloat16)])
    b = torch.cat([b, torch.tensor(sb, dtype=torch.float64).to(torch.bfloat16)])
    ref = (a + b).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.vector_add(a, b, "bf16"), ref)


def test_vector_add_exact_identities():
    x = np.random.default_rng(14).standard_normal(1000).astype(np.float32)
    z = np.zeros_like(x)
    assert np.array_equal(oracle.vector_add(x, z, "f32"), x.view(np.uint32))   # x + 0 = x
    s = oracle.vector_add(x, -x, "f32")                                           # x + (-x) = +0
    assert np.array_equal(s, np.zeros_like(s))
    assert np.array_equal(oracle.vector_add(x, x, "f32"), (2 * x).view(np.uint32))  # x + x = 2x exactly


# --------------------------------------------------------------------------
# standalone row softmax
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_softmax_rows_sum_to_one_and_keep_order(dtype):
    x = torch.randn(37, 300, generator=torch.Generator().manual_seed(15)).to(
        {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[dtype])
    y = oracle.softmax(x, 37, 300, dtype, alpha=0.7)
    assert np.allclose(y.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    xd = x.double().numpy()
    assert np.array_equal(np.argsort(y, axis=1, kind="stable"), np.argsort(xd, axis=1, kind="stable"))


def test_softmax_closed_forms():
    z = np.zeros((3, 64), dtype=np.float32)
    assert np.allclose(oracle.softmax(z, 3, 64, "f32"), 1 / 64, rtol=1e-15, atol=0)  # uniform rows
    one = np.array([[5.0], [-3.0]], dtype=np.float32)
    assert np.array_equal(oracle.softmax(one, 2, 1, "f32"), np.ones((2, 1)))          # single column
    ab = np.array([[1.5, -0.25]], dtype=np.float32)
    y = oracle.softmax(ab, 1, 2, "f32", alpha=2.0)                                      # logistic of the gap
    d = 2.0 * (1.5 + 0.25)
    assert np.allclose(y[0], [1 / (1 + math.exp(-d)), 1 / (1 + math.exp(d))], rtol=1e-15)


def test_softmax_shift_invariance():
    rng = np.random.default_rng(16)
    x = rng.integers(-20, 20, (8, 50)).astype(np.float32)
    y0 = oracle.softmax(x, 8, 50, "f32")
    y1 = oracle.softmax(x + np.float32(7), 8, 50, "f32")  # exact shift of integers
    assert np.allclose(y0, y1, rtol=1e-14, atol=0)


def test_softmax_equals_gemm_epilogue_with_identity():
    # X . I through the (separately pinned) GEMM oracle's softmax epilogue
    n = 48
    x = torch.randn(20, n, generator=torch.Generator().manual_seed(17)).to(torch.float16)
    eye = torch.eye(n, dtype=torch.float16)
    y_gemm = oracle.gemm(x, eye, None, 20, n, n, "f16", "softmax", alpha=0.5)
    y = oracle.softmax(x, 20, n, "f16", alpha=0.5)
    assert np.allclose(y, y_gemm, rtol=1e-14, atol=0)


def test_bad_arguments_rejected():
    with pytest.raises((ValueError, KeyError)):
        oracle.round_to([1.0], "f64")
    with pytest.raises(ValueError):
        oracle.vector_add(np.zeros(3, np.float32), np.zeros(4, np.float32), "f32")
    with pytest.raises(ValueError):
        oracle.softmax(np.zeros(6, np.float32), 2, 4, "f32")
