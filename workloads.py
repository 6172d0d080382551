"""Seeded synthetic inputs for the fused-epilogue GEMM workloads.

This module is shared by the tests, the benchmark and the smoke check.  It
holds no arithmetic of the method itself: it only draws random numbers, scales
them and rounds them to the input dtype.  Both the GPU path and the CPU oracle
consume exactly the tensors produced here.

Recipe (the same for every workload):
  * draw fp32 with ``torch.Generator('cpu').manual_seed(seed)``:
    ``torch.randn`` for N(0, 1), ``torch.rand * 2 - 1`` for U[-1, 1];
  * multiply by the fp32 scale (``1/sqrt(K)`` for the GEMM operands of the
    2048^3 and 8192^3 workloads, 1 otherwise);
  * round to fp16 / bf16 with ``Tensor.to`` (round to nearest even).

Sampled comparison positions come from ``torch.randperm(M*N)`` under their own
seed (without replacement), then ``(i, j) = (idx // N, idx % N)``.

The two bandwidth-bound kernels (vector addition, standalone row softmax) use
the same ``draw`` on their own seeds (``STREAM_WORKLOADS``).

The TileLang pages measure on synthetic matrices only (no dataset or public
benchmark suite is involved), so these stand in for nothing external.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dtype: str              # "f16" | "bf16"
    epilogue: str           # "none" | "bias" | "relu" | "gelu" | "softmax"
    dist: str               # "uniform" (U[-1,1]) | "normal" (N(0,1))
    scale: float            # multiplier applied to A and B draws (fp32)
    seeds: tuple            # (seed_A, seed_B, seed_bias or None, seed_sample or None)
    b_col_major: bool = False
    alpha: float = 1.0
    sample: int = 0         # 0: compare in full, else number of sampled outputs
    description: str = field(default="", compare=False)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def has_bias(self) -> bool:
        return self.epilogue in ("bias", "relu", "gelu")

    @property
    def out_dtype(self) -> str:
        return "f32" if self.epilogue == "softmax" else self.dtype

    def min_bytes(self) -> int:
        """Algorithmic HBM bytes: A, B and bias read once, C written once."""
        e = 2
        out = 4 if self.epilogue == "softmax" else 2
        return e * (self.M * self.K + self.K * self.N + (self.N if self.has_bias else 0)) + out * self.M * self.N


WORKLOADS = {
    "C1": Workload("C1", 64, 64, 64, "f16", "none", "uniform", 1.0, (101, 102, None, None),
                   description="64^3 fp16 U[-1,1], no epilogue"),
    "C2": Workload("C2", 2048, 2048, 2048, "f16", "none", "normal", 1.0 / math.sqrt(2048), (201, 202, None, None),
                   description="2048^3 fp16 N(0,1)/sqrt(2048), no epilogue"),
    "C3": Workload("C3", 2048, 2048, 2048, "f16", "gelu", "normal", 1.0 / math.sqrt(2048), (201, 202, 203, None),
                   description="2048^3 fp16 N(0,1)/sqrt(2048) + bias[N] N(0,1), GELU(acc+bias) erf form"),
    "C4a": Workload("C4a", 8192, 8192, 8192, "bf16", "relu", "normal", 1.0 / math.sqrt(8192),
                    (401, 402, 403, 404), sample=65536,
                    description="8192^3 bf16 N(0,1)/sqrt(8192) + bias[N] N(0,1), ReLU(acc+bias)"),
    "C4b": Workload("C4b", 3000, 5000, 1000, "bf16", "relu", "normal", 1.0 / math.sqrt(8192),
                    (411, 412, 413, None),
                    description="3000x5000x1000 bf16, same distributions as the 8192^3 case, ReLU(acc+bias)"),
    "C5": Workload("C5", 4096, 1024, 128, "f16", "softmax", "normal", 1.0, (501, 502, None, None),
                   b_col_major=True, alpha=float(torch.tensor(1.0 / math.sqrt(128), dtype=torch.float32)),
                   description="A 4096x128, B col-major 128x1024 (stored 1024x128), fp16 N(0,1), "
                               "row softmax of acc/sqrt(128), fp32 out"),
}

TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def draw(shape, seed: int, dist: str, scale: float, dtype: str) -> torch.Tensor:
    """fp32 draw under ``seed``, scaled in fp32, rounded once to ``dtype`` (CPU tensor)."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    if dist == "normal":
        x = torch.randn(shape, generator=g, dtype=torch.float32)
    elif dist == "uniform":
        x = torch.rand(shape, generator=g, dtype=torch.float32) * 2.0 - 1.0
    else:
        raise ValueError(dist)
    if scale != 1.0:
        x = x * torch.tensor(scale, dtype=torch.float32)
    return x.to(TORCH_DTYPES[dtype])


def make_inputs(w: Workload):
    """(A, B, bias) CPU tensors.  A is M x K; B is K x N, or N x K when b_col_major."""
    sa, sb, sbias, _ = w.seeds
    A = draw((w.M, w.K), sa, w.dist, w.scale, w.dtype)
    B = draw((w.N, w.K) if w.b_col_major else (w.K, w.N), sb, w.dist, w.scale, w.dtype)
    bias = draw((w.N,), sbias, "normal", 1.0, w.dtype) if w.has_bias else None
    return A, B, bias


def sample_positions(M: int, N: int, count: int, seed: int):
    """``count`` distinct output positions (rows, cols), drawn without replacement."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    idx = torch.randperm(M * N, generator=g)[:count]
    return (idx // N).numpy(), (idx % N).numpy()


def random_matrix(shape, seed: int, dtype: str, dist: str = "normal", scale: float = 1.0) -> torch.Tensor:
    """Generic seeded operand for parity sweeps at arbitrary shapes."""
    return draw(shape, seed, dist, scale, dtype)


# ---- the bandwidth-bound kernels ---------------------------------------------

ELEMENT_BYTES = {"f16": 2, "bf16": 2, "f32": 4}


@dataclass(frozen=True)
class StreamWorkload:
    name: str
    kind: str               # "vector_add" (n = rows * cols elements) | "row_softmax" (rows x cols)
    rows: int
    cols: int
    dtype: str              # "f16" | "bf16" | "f32"
    dist: str
    scale: float
    seeds: tuple            # (seed_A or seed_X, seed_B or None, seed_sample)
    alpha: float = 1.0
    description: str = field(default="", compare=False)

    @property
    def n(self) -> int:
        return self.rows * self.cols

    def min_bytes(self) -> int:
        """Algorithmic HBM bytes: every input read once, every output written once."""
        e = ELEMENT_BYTES[self.dtype]
        if self.kind == "vector_add":
            return 3 * e * self.n
        return (e + 4) * self.n  # X in its dtype, Y in fp32


STREAM_WORKLOADS = {
    "V1": StreamWorkload("V1", "vector_add", 1, 1 << 22, "f32", "uniform", 1.0, (601, 602, 603),
                         description="vector add, 2^22 fp32 U[-1,1] (48 MiB moved: fits the 256 MB MALL)"),
    "V2": StreamWorkload("V2", "vector_add", 1, 1 << 28, "f32", "uniform", 1.0, (611, 612, 613),
                         description="vector add, 2^28 fp32 U[-1,1] (3 GiB moved: HBM-resident)"),
    "S1": StreamWorkload("S1", "row_softmax", 16384, 4096, "f16", "normal", 1.0, (621, None, 623),
                         description="row softmax, X 16384x4096 fp16 N(0,1), alpha 1, fp32 out"),
}


def make_stream_inputs(w: StreamWorkload):
    """(A, B) for a vector add (flat CPU tensors of n elements), or (X, None) for a
    row softmax (rows x cols)."""
    sa, sb, _ = w.seeds
    if w.kind == "vector_add":
        return draw((w.n,), sa, w.dist, w.scale, w.dtype), draw((w.n,), sb, w.dist, w.scale, w.dtype)
    return draw((w.rows, w.cols), sa, w.dist, w.scale, w.dtype), None


# ---- attention forward -----------------------------------------------------------

@dataclass(frozen=True)
class AttnWorkload:
    name: str
    B: int
    H: int
    N: int
    D: int
    dtype: str
    causal: bool
    seeds: tuple            # (seed_Q, seed_K, seed_V, seed_sample)
    description: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        """1/sqrt(D) as the fp32 value both sides receive."""
        return float(torch.tensor(1.0 / math.sqrt(self.D), dtype=torch.float32))

    @property
    def flops(self) -> int:
        """4 D FLOPs (two products) per visible (query, key) pair."""
        pairs = self.N * (self.N + 1) // 2 if self.causal else self.N * self.N
        return 4 * self.B * self.H * self.D * pairs

    def min_bytes(self) -> int:
        """Q, K, V read once, O written once."""
        return 4 * self.B * self.H * self.N * self.D * ELEMENT_BYTES[self.dtype]


ATTN_WORKLOADS = {
    "A1": AttnWorkload("A1", 4, 16, 4096, 128, "f16", False, (701, 702, 703, 704),
                       description="attention fwd, B=4 H=16 N=4096 D=128 fp16 N(0,1), non-causal, scale 1/sqrt(128)"),
    "A2": AttnWorkload("A2", 4, 16, 4096, 128, "f16", True, (711, 712, 713, 714),
                       description="attention fwd, B=4 H=16 N=4096 D=128 fp16 N(0,1), causal, scale 1/sqrt(128)"),
    "A3": AttnWorkload("A3", 4, 32, 4096, 64, "bf16", False, (721, 722, 723, 724),
                       description="attention fwd, B=4 H=32 N=4096 D=64 bf16 N(0,1), non-causal, scale 1/sqrt(64)"),
}


def make_attention_inputs(w: AttnWorkload):
    """(Q, K, V) CPU tensors of shape (B, H, N, D), N(0,1) rounded to the dtype."""
    shape = (w.B, w.H, w.N, w.D)
    return tuple(draw(shape, s, "normal", 1.0, w.dtype) for s in w.seeds[:3])
