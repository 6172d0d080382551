"""CPU oracle for Y = epilogue(alpha * A.B + bias), the tutorial's vector
addition and row softmax, and attention forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it and
shares no code with it (``oracle/oracle.c`` has its own decoders, enums and
epilogue formulas).

What it computes (fp64, unrounded), following the TileLang tutorial pages:

* "TileLang: Criando Kernels de GPU de Alto Desempenho com Tensor Cores,
  FlashAttention e Autotuning" (noticiai.com.br): section "GEMM com Tensor
  Cores" for the product, "GEMM com epilogo fundido" for ReLU / bias / GELU on
  the accumulator, "Softmax por linha e FlashAttention" for the row softmax
  (max, subtract, exponentiate, normalise);
* the edgex.exchange page on the TileLang Python DSL, paragraph on the fused
  epilogue (bias + GELU folded into the accumulator; row softmax);
* "Designing High-Performance GPU Kernels with TileLang ..." (spaxe.top),
  paragraph on the softmax applied in the GEMM epilogue.

Steps: decode every fp16/bf16 input exactly to fp64; ``acc = sum_k a_ik b_kj``
in k order with one fp64 accumulator; ``x = alpha*acc + bias_j`` (bias indexed
by column, broadcast over rows); then none / ReLU ``max(x, 0)`` /
GELU ``0.5 x (1 + erf(x / sqrt 2))`` / row softmax ``exp(x - max) / sum``.

Attention (what the tutorial's FlashAttention forward computes, section
"Softmax por linha e FlashAttention" and the other pages' FlashAttention
paragraphs): per query row, ``s_j = scale * q . k_j`` over all keys (causal:
keys j <= i), softmax over j, ``o = sum_j p_j v_j``; the plain definition, not
the online reformulation.  Pins in ``tests/test_oracle_attention.py``.

Pins: every function here is checked in ``tests/test_oracle.py`` against
closed forms, exact rational arithmetic, library routines and textbook
values; none is "parity unpinned".
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPES = {"f16": 0, "fp16": 0, "float16": 0, "bf16": 1, "bfloat16": 1, "f32": 2, "fp32": 2, "float32": 2}
EPILOGUES = {"none": 0, "bias": 1, "relu": 2, "bias_relu": 2, "gelu": 3, "bias_gelu": 3, "softmax": 4}

_lib = None


def build() -> str:
    """Compile oracle.c into liboracle.so (plain gcc, OpenMP, no fp contraction)."""
    cmd = [
        "gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
        "-fPIC", "-shared", _SRC, "-o", _LIB, "-lm",
    ]
    subprocess.run(cmd, check=True)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    ci = ctypes.c_int
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_act.argtypes = [f64p, f64p, i64, ci]
    lib.oracle_act.restype = ci
    lib.oracle_gemm.argtypes = [u16p, u16p, u16p, f64p, i64, i64, i64, ci, ci, ci, ctypes.c_double, ci]
    lib.oracle_gemm.restype = ci
    lib.oracle_gemm_sampled.argtypes = [u16p, u16p, u16p, i64p, i64p, i64, f64p, i64, i64, i64, ci, ci,
                                        ci, ctypes.c_double, ci]
    lib.oracle_gemm_sampled.restype = ci
    lib.oracle_max_threads.argtypes = [ci]
    lib.oracle_max_threads.restype = ci
    vp = ctypes.c_void_p
    lib.oracle_f32_to_f64.argtypes = [ctypes.c_uint32]
    lib.oracle_f32_to_f64.restype = ctypes.c_double
    lib.oracle_round.argtypes = [f64p, vp, i64, ci]
    lib.oracle_round.restype = ci
    lib.oracle_vector_add.argtypes = [vp, vp, vp, i64, ci]
    lib.oracle_vector_add.restype = ci
    lib.oracle_softmax.argtypes = [vp, f64p, i64, i64, ci, ctypes.c_double, ci]
    lib.oracle_softmax.restype = ci
    lib.oracle_attention_rows.argtypes = [u16p, u16p, u16p, f64p, i64, i64, i64, i64, ci, ci, ctypes.c_double,
                                          i64p, i64, ci]
    lib.oracle_attention_rows.restype = ci
    lib.oracle_attention.argtypes = [u16p, u16p, u16p, f64p, i64, i64, i64, i64, ci, ci, ctypes.c_double, ci]
    lib.oracle_attention.restype = ci
    _lib = lib
    return lib


def _bits(x) -> np.ndarray:
    """uint16 view of fp16/bf16 data given as a torch tensor or numpy array."""
    if x is None:
        return None
    if hasattr(x, "view") and hasattr(x, "dtype") and "torch" in type(x).__module__:
        import torch
        x = x.detach().cpu().contiguous().view(torch.int16).numpy()
    a = np.ascontiguousarray(x)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"expected 16-bit storage, got {a.dtype}")
    return a


def _ptr(a, ctype):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctype))


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def threads_used(nthreads: int | None = None) -> int:
    return _load().oracle_max_threads(nthreads or default_threads())


def f16_to_f64(bits: int) -> float:
    return _load().oracle_f16_to_f64(bits)


def bf16_to_f64(bits: int) -> float:
    return _load().oracle_bf16_to_f64(bits)


def decode(bits, dtype: str) -> np.ndarray:
    """Exact fp64 values of an array of fp16/bf16 bit patterns."""
    b = _bits(bits).ravel()
    f = f16_to_f64 if DTYPES[dtype] == 0 else bf16_to_f64
    return np.array([f(int(v)) for v in b], dtype=np.float64)


def act(x, epilogue: str) -> np.ndarray:
    """Elementwise epilogue activation (none / bias / relu / gelu) in fp64."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    rc = _load().oracle_act(_ptr(x, ctypes.c_double), _ptr(y, ctypes.c_double), x.size, EPILOGUES[epilogue])
    if rc != 0:
        raise ValueError(f"oracle_act rejected epilogue {epilogue!r}")
    return y


def gemm(A, B, bias, M: int, N: int, K: int, dtype: str, epilogue: str, b_col_major: bool = False,
         alpha: float = 1.0, threads: int | None = None) -> np.ndarray:
    """Full fp64 result Y (M x N).  A: M*K, B: K*N (or N*K if b_col_major), bias: N or None."""
    a, b, c = _bits(A), _bits(B), _bits(bias)
    if a.size != M * K or b.size != K * N or (c is not None and c.size != N):
        raise ValueError("operand sizes do not match M, N, K")
    y = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_gemm(_ptr(a, ctypes.c_uint16), _ptr(b, ctypes.c_uint16), _ptr(c, ctypes.c_uint16),
                             _ptr(y, ctypes.c_double), M, N, K, DTYPES[dtype], EPILOGUES[epilogue],
                             int(bool(b_col_major)), float(alpha), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_gemm rejected its arguments")
    return y


def gemm_sampled(A, B, bias, rows, cols, M: int, N: int, K: int, dtype: str, epilogue: str,
                 b_col_major: bool = False, alpha: float = 1.0, threads: int | None = None) -> np.ndarray:
    """Y[rows[s], cols[s]] for each sample s, each as its own fp64 dot product."""
    a, b, c = _bits(A), _bits(B), _bits(bias)
    if a.size != M * K or b.size != K * N or (c is not None and c.size != N):
        raise ValueError("operand sizes do not match M, N, K")
    r = np.ascontiguousarray(rows, dtype=np.int64)
    q = np.ascontiguousarray(cols, dtype=np.int64)
    if r.shape != q.shape:
        raise ValueError("rows and cols differ in length")
    y = np.empty(r.size, dtype=np.float64)
    rc = _load().oracle_gemm_sampled(_ptr(a, ctypes.c_uint16), _ptr(b, ctypes.c_uint16), _ptr(c, ctypes.c_uint16),
                                     _ptr(r, ctypes.c_int64), _ptr(q, ctypes.c_int64), r.size,
                                     _ptr(y, ctypes.c_double), M, N, K, DTYPES[dtype], EPILOGUES[epilogue],
                                     int(bool(b_col_major)), float(alpha), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_gemm_sampled rejected its arguments")
    return y


# ---- the bandwidth-bound kernels of the tutorial: vector add, row softmax ----

def _storage(x, dtype: str) -> np.ndarray:
    """Raw element bits of a torch tensor / numpy array: uint16 for fp16 and
    bf16, uint32 for fp32."""
    if DTYPES[dtype] == 2:
        if hasattr(x, "view") and "torch" in type(x).__module__:
            import torch
            x = x.detach().cpu().contiguous().view(torch.int32).numpy()
        a = np.ascontiguousarray(x)
        if a.dtype == np.float32 or a.dtype == np.int32:
            a = a.view(np.uint32)
        if a.dtype != np.uint32:
            raise TypeError(f"expected 32-bit storage, got {a.dtype}")
        return a
    return _bits(x)


def f32_to_f64(bits: int) -> float:
    return _load().oracle_f32_to_f64(bits)


def round_to(x, dtype: str) -> np.ndarray:
    """Bit patterns of the dtype values nearest to fp64 values x (ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint32 if DTYPES[dtype] == 2 else np.uint16)
    if _load().oracle_round(_ptr(x, ctypes.c_double), out.ctypes.data, x.size, DTYPES[dtype]) != 0:
        raise ValueError("oracle_round rejected its arguments")
    return out


def vector_add(A, B, dtype: str) -> np.ndarray:
    """C = A + B, correctly rounded to dtype, as bit patterns (uint16 / uint32)."""
    a, b = _storage(A, dtype).ravel(), _storage(B, dtype).ravel()
    if a.size != b.size:
        raise ValueError("A and B differ in length")
    c = np.empty_like(a)
    if _load().oracle_vector_add(a.ctypes.data, b.ctypes.data, c.ctypes.data, a.size, DTYPES[dtype]) != 0:
        raise ValueError("oracle_vector_add rejected its arguments")
    return c


def softmax(X, rows: int, cols: int, dtype: str, alpha: float = 1.0, threads: int | None = None) -> np.ndarray:
    """Y = row softmax of alpha * X (rows x cols), fp64, unrounded."""
    x = _storage(X, dtype).ravel()
    if x.size != rows * cols:
        raise ValueError("X does not have rows * cols elements")
    y = np.empty((rows, cols), dtype=np.float64)
    if _load().oracle_softmax(x.ctypes.data, _ptr(y, ctypes.c_double), rows, cols, DTYPES[dtype], float(alpha),
                              threads or default_threads()) != 0:
        raise ValueError("oracle_softmax rejected its arguments")
    return y


def _attention_args(Q, K, V, B, H, N, D):
    q, k, v = _bits(Q).ravel(), _bits(K).ravel(), _bits(V).ravel()
    if not (q.size == k.size == v.size == B * H * N * D):
        raise ValueError("Q, K, V must each hold B*H*N*D elements")
    return q, k, v


def attention(Q, K, V, B: int, H: int, N: int, D: int, dtype: str, causal: bool = False,
              scale: float | None = None, threads: int | None = None) -> np.ndarray:
    """O = softmax(scale * Q K^T [causal mask]) V per (batch, head); [B][H][N][D]
    row-major inputs, fp64 output of shape (B, H, N, D).  scale defaults to 1/sqrt(D)."""
    q, k, v = _attention_args(Q, K, V, B, H, N, D)
    o = np.empty((B, H, N, D), dtype=np.float64)
    sc = 1.0 / np.sqrt(D) if scale is None else float(scale)
    rc = _load().oracle_attention(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16),
                                  _ptr(o, ctypes.c_double), B, H, N, D, DTYPES[dtype], int(bool(causal)), sc,
                                  threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_attention rejected its arguments ({rc})")
    return o


def attention_rows(Q, K, V, rows, B: int, H: int, N: int, D: int, dtype: str, causal: bool = False,
                   scale: float | None = None, threads: int | None = None) -> np.ndarray:
    """The output rows O[r] for flat query rows r = (b*H + h)*N + i; shape (len(rows), D)."""
    q, k, v = _attention_args(Q, K, V, B, H, N, D)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    o = np.empty((r.size, D), dtype=np.float64)
    sc = 1.0 / np.sqrt(D) if scale is None else float(scale)
    rc = _load().oracle_attention_rows(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                                       _ptr(v, ctypes.c_uint16), _ptr(o, ctypes.c_double), B, H, N, D,
                                       DTYPES[dtype], int(bool(causal)), sc, _ptr(r, ctypes.c_int64), r.size,
                                       threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_attention_rows rejected its arguments ({rc})")
    return o
