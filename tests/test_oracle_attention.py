"""Pins of the attention oracle (CPU only).

The oracle is the plain definition of attention (see oracle/oracle.c).  These
tests tie it to facts that hold independently of how it is written, each
chosen so that a plausible mistake fails one of them:

* uniform scores (Q = 0 or scale = 0): every output row is the mean of the
  visible value rows -- all of them, or the prefix 0..i when causal (a wrong
  mask direction, an off-by-one in the mask or a missing normalisation fails);
* causal row 0 is V[0] exactly, and a causal row never depends on later keys
  or values (mask direction);
* two keys: the output is the logistic blend sigma(s0 - s1) v0 + sigma(s1 - s0) v1
  (closed form, scores exact from small integers);
* a very large scale turns softmax into argmax: the output is the value row of
  the highest-scoring key (swapping the roles of Q and K picks other rows);
* adding one vector to every key leaves the output unchanged (the softmax runs
  over keys, per query -- normalising over the wrong axis fails);
* permuting keys and values together leaves the output unchanged; permuting
  queries permutes output rows (index / stride mistakes);
* linearity in V and convexity (every output lies within the range of V);
* each (batch, head) slice equals the oracle run on that slice alone, and the
  rows mode equals the full mode bit for bit.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _h(x):
    """fp16 tensor from exactly representable values."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float64)).to(torch.float16)
    assert np.array_equal(t.double().numpy(), np.asarray(x, dtype=np.float64)), "not exact in fp16"
    return t


def _rand(shape, seed, dtype=torch.float16, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype)


def _dt(t):
    return "f16" if t.dtype == torch.float16 else "bf16"


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_scores_give_prefix_or_full_means(causal):
    B, H, N, D = 2, 3, 7, 5
    rng = np.random.default_rng(1)
    V = _h(rng.integers(-8, 9, (B, H, N, D)))
    Q = torch.zeros((B, H, N, D), dtype=torch.float16)
    K = _rand((B, H, N, D), 2)
    o = oracle.attention(Q, K, V, B, H, N, D, "f16", causal=causal)
    v = V.double().numpy()
    for i in range(N):
        want = v[:, :, : i + 1].mean(axis=2) if causal else v.mean(axis=2)
        assert np.allclose(o[:, :, i], want, rtol=0, atol=1e-13)
    # scale = 0 makes every score equal too, whatever Q and K are
    o0 = oracle.attention(_rand((B, H, N, D), 3), K, V, B, H, N, D, "f16", causal=causal, scale=0.0)
    assert np.allclose(o0, o, rtol=0, atol=1e-13)


def test_causal_first_row_and_prefix_independence():
    B, H, N, D = 1, 2, 9, 8
    Q, K, V = _rand((B, H, N, D), 4), _rand((B, H, N, D), 5), _rand((B, H, N, D), 6)
    o = oracle.attention(Q, K, V, B, H, N, D, "f16", causal=True)
    assert np.array_equal(o[:, :, 0], V[:, :, 0].double().numpy())
    K2, V2 = K.clone(), V.clone()
    K2[:, :, 5:] = _rand((B, H, N - 5, D), 7)
    V2[:, :, 5:] = _rand((B, H, N - 5, D), 8)
    o2 = oracle.attention(Q, K2, V2, B, H, N, D, "f16", causal=True)
    assert np.array_equal(o2[:, :, :5], o[:, :, :5])  # rows 0..4 see keys 0..4 only
    assert not np.allclose(o2[:, :, 5:], o[:, :, 5:])


def test_two_keys_logistic_closed_form():
    D = 4
    Q = _h([[[[1, 2, 0, -1], [0.5, -3, 2, 1]]]])          # B=1, H=1, N=2
    K = _h([[[[2, -1, 1, 0], [-1, 1, 0.5, 3]]]])
    V = _h([[[[1, 0, -2, 4], [-3, 5, 0.25, 1]]]])
    scale = 0.375  # exact in binary
    o = oracle.attention(Q, K, V, 1, 1, 2, D, "f16", causal=False, scale=scale)
    q, k, v = Q[0, 0].double().numpy(), K[0, 0].double().numpy(), V[0, 0].double().numpy()
    for i in range(2):
        s0 = float(Fraction(scale) * sum(Fraction(a) * Fraction(b) for a, b in zip(q[i], k[0])))
        s1 = float(Fraction(scale) * sum(Fraction(a) * Fraction(b) for a, b in zip(q[i], k[1])))
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        want = w0 * v[0] + (1.0 - w0) * v[1]
        assert np.allclose(o[0, 0, i], want, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_large_scale_selects_the_argmax_key(causal):
    B, H, N, D = 1, 1, 6, 3
    rng = np.random.default_rng(9)
    Q = _h(rng.integers(-3, 4, (B, H, N, D)))
    K = _h(rng.integers(-3, 4, (B, H, N, D)))
    V = _h(rng.integers(-8, 9, (B, H, N, D)))
    q, k, v = Q[0, 0].double().numpy(), K[0, 0].double().numpy(), V[0, 0].double().numpy()
    s = q @ k.T  # exact (small integers)
    o = oracle.attention(Q, K, V, B, H, N, D, "f16", causal=causal, scale=1e4)
    checked = 0
    for i in range(N):
        row = s[i, : i + 1] if causal else s[i]
        top = np.flatnonzero(row == row.max())
        if top.size != 1:
            continue  # tie: the blend of the tied rows, not checked here
        assert np.allclose(o[0, 0, i], v[top[0]], rtol=0, atol=1e-12)
        checked += 1
    assert checked >= 3


@pytest.mark.parametrize("causal", [False, True])
def test_shifting_every_key_by_one_vector_changes_nothing(causal):
    B, H, N, D = 1, 2, 8, 4
    rng = np.random.default_rng(11)
    Q = _h(rng.integers(-4, 5, (B, H, N, D)) / 4)
    K = _h(rng.integers(-4, 5, (B, H, N, D)) / 4)
    V = _rand((B, H, N, D), 12)
    u = rng.integers(-4, 5, (B, H, 1, D)) / 2
    K2 = _h(K.double().numpy() + u)  # exact: quarters and halves of small integers
    o = oracle.attention(Q, K, V, B, H, N, D, "f16", causal=causal, scale=0.5)
    o2 = oracle.attention(Q, K2, V, B, H, N, D, "f16", causal=causal, scale=0.5)
    assert np.allclose(o, o2, rtol=0, atol=1e-12)
    # shifting one query's scores is not the same as shifting keys: a shift of
    # the *values* of one key moves the output (sanity of the test itself)
    V2 = V.clone()
    V2[:, :, 0] += 1
    assert not np.allclose(oracle.attention(Q, K, V2, B, H, N, D, "f16", causal=causal, scale=0.5), o)


def test_noncausal_permutations():
    B, H, N, D = 1, 1, 10, 6
    Q, K, V = _rand((B, H, N, D), 13), _rand((B, H, N, D), 14), _rand((B, H, N, D), 15)
    o = oracle.attention(Q, K, V, B, H, N, D, "f16")
    perm = torch.randperm(N, generator=torch.Generator().manual_seed(16))
    ok = oracle.attention(Q, K[:, :, perm], V[:, :, perm], B, H, N, D, "f16")
    assert np.allclose(ok, o, rtol=0, atol=1e-13)  # sum order changes, nothing else
    oq = oracle.attention(Q[:, :, perm], K, V, B, H, N, D, "f16")
    assert np.array_equal(oq, o[:, :, perm.numpy()])


@pytest.mark.parametrize("causal", [False, True])
def test_linear_in_values_and_convex(causal):
    B, H, N, D = 1, 2, 12, 8
    rng = np.random.default_rng(17)
    Q, K = _rand((B, H, N, D), 18, torch.bfloat16), _rand((B, H, N, D), 19, torch.bfloat16)
    V1 = rng.integers(-64, 65, (B, H, N, D)) / 8
    V2 = rng.integers(-64, 65, (B, H, N, D)) / 8
    to_bf = lambda x: torch.as_tensor(x).to(torch.bfloat16)  # noqa: E731  (exact: 7-bit integers / 8)
    o1 = oracle.attention(Q, K, to_bf(V1), B, H, N, D, "bf16", causal=causal)
    o2 = oracle.attention(Q, K, to_bf(V2), B, H, N, D, "bf16", causal=causal)
    o12 = oracle.attention(Q, K, to_bf(V1 + V2), B, H, N, D, "bf16", causal=causal)
    assert np.allclose(o12, o1 + o2, rtol=0, atol=1e-12)
    lo, hi = V1.min(axis=2, keepdims=True), V1.max(axis=2, keepdims=True)
    assert np.all(o1 >= lo - 1e-12) and np.all(o1 <= hi + 1e-12)


def test_slices_rows_mode_and_trivial_shapes():
    B, H, N, D = 2, 3, 5, 4
    Q, K, V = _rand((B, H, N, D), 20), _rand((B, H, N, D), 21), _rand((B, H, N, D), 22)
    for causal in (False, True):
        o = oracle.attention(Q, K, V, B, H, N, D, "f16", causal=causal)
        for b in range(B):
            for h in range(H):
                s = oracle.attention(Q[b, h].contiguous(), K[b, h].contiguous(), V[b, h].contiguous(), 1, 1, N, D,
                                     "f16", causal=causal)
                assert np.array_equal(s[0, 0], o[b, h])
        rows = np.array([0, 7, 13, 29, B * H * N - 1])
        r = oracle.attention_rows(Q, K, V, rows, B, H, N, D, "f16", causal=causal)
        assert np.array_equal(r, o.reshape(-1, D)[rows])
    # N = 1: the single value row, whatever the scores
    o1 = oracle.attention(Q[:, :, :1].contiguous(), K[:, :, :1].contiguous(), V[:, :, :1].contiguous(), B, H, 1, D,
                          "f16")
    assert np.array_equal(o1, V[:, :, :1].double().numpy())
    # N = 0: nothing to compute
    e = torch.empty((B, H, 0, D), dtype=torch.float16)
    assert oracle.attention(e, e, e, B, H, 0, D, "f16").shape == (B, H, 0, D)


def test_default_scale_is_inverse_sqrt_of_head_dim():
    B, H, N, D = 1, 1, 6, 16
    Q, K, V = _rand((B, H, N, D), 23), _rand((B, H, N, D), 24), _rand((B, H, N, D), 25)
    assert np.array_equal(oracle.attention(Q, K, V, B, H, N, D, "f16"),
                          oracle.attention(Q, K, V, B, H, N, D, "f16", scale=0.25))


def test_bad_arguments_rejected():
    z = torch.zeros((1, 1, 4, 4), dtype=torch.float16)
    with pytest.raises(ValueError):
        oracle.attention(z, z, z, 1, 1, 4, 5, "f16")        # sizes do not match
    with pytest.raises(ValueError):
        oracle.attention_rows(z, z, z, [16], 1, 1, 4, 4, "f16")  # row out of range
    with pytest.raises(ValueError):
        oracle.attention_rows(z, z, z, [-1], 1, 1, 4, 4, "f16")
