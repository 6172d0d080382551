"""CPU checks of the constants the GPU epilogue uses (no GPU needed).

The GELU epilogue evaluates erfc(z) ~= t exp(-z^2 + P(t)), t = 1/(1 + z/2),
with a cubic P fitted for this library.  The natural-log coefficients are
read from the kernel source and the stated bounds (relative error of erfc
below 1.2e-4 on z in [0, 4.3] and below 9.4e-4 on [0, 9]) are checked in fp64
against scipy.special.erfc; the folded fp32 constants the kernel actually
uses are checked against the natural-log ones; the fp32 evaluation of the
whole GELU is checked against x Phi(x), and the bounds against half an ulp
of the output formats, so that a rounded result is at most one ulp from the
correctly rounded one.
"""

import math
import os
import re

import numpy as np
from scipy.special import erfc, ndtr

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "dense_gemm_epilogues_tiled_amd",
                   "csrc", "device.hpp")


def _natural_coefficients():
    text = open(SRC).read()
    m = re.search(r"Natural-log coefficients of P \(t\^0 \.\. t\^3\), as fitted:\s*//\s*([^\n]+)", text)
    assert m, "coefficient comment not found"
    return [float(v) for v in m.group(1).split(",")]


def _folded_constants():
    body = open(SRC).read().split("float gelu_erf(float x)")[1].split("\n}")[0]
    return [float(v) for v in re.findall(r"(-?\d+\.\d+)f", body)]


# half an ulp, relative, at its smallest (a value just below a power of two)
HALF_ULP = {"f16": 2.0 ** -12, "bf16": 2.0 ** -9}


def test_erfc_fit_bound():
    c = _natural_coefficients()
    assert len(c) == 4
    z = np.linspace(0.0, 9.0, 400001)
    t = 1.0 / (1.0 + z / 2.0)
    approx = t * np.exp(-z * z + np.polyval(c[::-1], t))
    rel = np.abs(approx / erfc(z) - 1.0)
    near = z <= 4.3
    assert rel[near].max() < 1.2e-4 < HALF_ULP["f16"]
    assert rel.max() < 9.4e-4 < HALF_ULP["bf16"]


def test_folded_constants_match():
    c = _natural_coefficients()
    l2e = math.log2(math.e)
    k = _folded_constants()
    # order in the source: 0.5/sqrt2, 1.0, then P2 from t^3 down to t^0,
    # then sqrt(log2e/2), then 0.0 (the max with zero)
    assert len(k) == 8
    assert abs(k[0] - 0.5 / math.sqrt(2)) < 1e-8 and k[1] == 1.0 and k[7] == 0.0
    p2 = k[2:6][::-1]  # t^0 .. t^3
    want = [l2e * v for v in c]
    want[0] -= 1.0
    for a, b in zip(p2, want):
        assert abs(a - b) <= 2e-7 * max(1.0, abs(b))
    assert abs(k[6] - math.sqrt(l2e / 2)) < 1e-7


def test_gelu_form_in_fp32_simulation():
    """The device sequence, replayed in fp32 with numpy, against x * Phi(x)."""
    k = [np.float32(v) for v in _folded_constants()]
    x = np.linspace(-10, 10, 200001).astype(np.float32)
    ax = np.abs(x)
    t = (np.float32(1) / (ax * k[0] + np.float32(1))).astype(np.float32)
    p = np.full_like(t, k[2])
    for cst in k[3:6]:
        p = (p * t + cst).astype(np.float32)
    zz = (ax * k[6]).astype(np.float32)
    q = (t * np.exp2((-zz * zz + p).astype(np.float64)).astype(np.float32)).astype(np.float32)
    g = (np.maximum(x, np.float32(0)) - ax * q).astype(np.float32)
    ref = x.astype(np.float64) * ndtr(x.astype(np.float64))
    keep = np.abs(ref) > 1e-30
    rel = np.abs(g[keep] - ref[keep]) / np.abs(ref[keep])
    xs = np.abs(x[keep])
    # every value an fp16 output resolves, within the fp16 budget; the tail, within bf16's
    assert rel[xs <= 6.1].max() < 1.3e-4 < HALF_ULP["f16"]
    assert rel.max() < 1.0e-3 < HALF_ULP["bf16"]
