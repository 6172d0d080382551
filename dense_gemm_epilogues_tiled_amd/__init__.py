"""Python binding of libtg.so, the gfx950 fused-epilogue GEMM library.

    C = epilogue(alpha * A.B + bias)      (see include/tg.h)

This module only marshals arguments: every step of the computation runs in
the HIP kernels of ``libtg.so``.  torch provides device memory and the
current stream.  The library is loaded after torch so that both use the same
HIP runtime instance.

Functions named ``tg_*`` mirror the C entry points one to one (they take raw
integers / pointers and return the status code).  ``gemm`` is the tensor-level
convenience wrapper: it checks device, dtype, shape and contiguity, allocates
the output if needed, and raises ``TgError`` on a non-zero status.
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must be imported before libtg.so: shared HIP runtime)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtg.so")

# ---- constants of include/tg.h --------------------------------------------
TG_OK = 0
TG_ERR_INVALID_ARG = -1
TG_ERR_UNSUPPORTED = -2
TG_ERR_MISALIGNED = -3
TG_ERR_HIP = -4

TG_DTYPE_F16 = 0
TG_DTYPE_BF16 = 1
TG_DTYPE_F32 = 2

TG_EPI_NONE = 0
TG_EPI_BIAS = 1
TG_EPI_BIAS_RELU = 2
TG_EPI_BIAS_GELU = 3
TG_EPI_SOFTMAX = 4

TG_KERNEL_GEMM = 0
TG_KERNEL_GEMM_SOFTMAX = 1

TG_SOFTMAX_MAX_N = 2048
TG_ROW_SOFTMAX_MAX_ROW_BYTES = 16384
TG_ATTN_MAX_SEQ = 1 << 20
TG_AUTOTUNE_NOALLOC_MAX_BYTES = 32 * 1024 * 1024 + 8192

EPILOGUES = {
    "none": TG_EPI_NONE, "bias": TG_EPI_BIAS, "relu": TG_EPI_BIAS_RELU, "bias_relu": TG_EPI_BIAS_RELU,
    "gelu": TG_EPI_BIAS_GELU, "bias_gelu": TG_EPI_BIAS_GELU, "softmax": TG_EPI_SOFTMAX,
}
DTYPES = {torch.float16: TG_DTYPE_F16, torch.bfloat16: TG_DTYPE_BF16}
STREAM_DTYPES = {torch.float16: TG_DTYPE_F16, torch.bfloat16: TG_DTYPE_BF16, torch.float32: TG_DTYPE_F32}


class tg_tile_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "id", "kind", "bm", "bn", "bk", "stages", "waves", "mfma_m", "mfma_n", "mfma_k", "wave_m", "wave_n",
        "group_m", "xcd_remap", "lds_bytes", "b_col_major")]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


class tg_gemm_args(ctypes.Structure):
    _fields_ = [
        ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("C", ctypes.c_void_p),
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("epilogue", ctypes.c_int32), ("b_col_major", ctypes.c_int32),
        ("alpha", ctypes.c_float), ("config_id", ctypes.c_int32), ("group_m", ctypes.c_int32),
        ("xcd_remap", ctypes.c_int32),
    ]


class tg_autotune_entry(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("b_col_major", ctypes.c_int32), ("kind", ctypes.c_int32),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("config", tg_tile_config),
                ("us", ctypes.c_float), ("candidates", ctypes.c_int32), ("valid", ctypes.c_int32)]

    def as_dict(self) -> dict:
        d = {n: getattr(self, n) for n, _ in self._fields_ if n != "config"}
        d["config"] = self.config.as_dict()
        return d


# Every function include/tg.h declares, with its ctypes signature.
_SIGNATURES = {
    "tg_gemm": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                               ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "tg_gemm_ex": (ctypes.c_int, [ctypes.POINTER(tg_gemm_args), ctypes.c_void_p]),
    "tg_gemm_query_config": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.POINTER(tg_tile_config)]),
    "tg_vector_add": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                     ctypes.c_void_p]),
    "tg_row_softmax": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                      ctypes.c_float, ctypes.c_void_p]),
    "tg_attention_fwd": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_float, ctypes.c_void_p]),
    "tg_gemm_autotune_workspace_size": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                                       ctypes.POINTER(ctypes.c_int64)]),
    "tg_gemm_autotune": (ctypes.c_int, [ctypes.POINTER(tg_gemm_args), ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                        ctypes.POINTER(tg_autotune_entry), ctypes.c_void_p]),
    "tg_gemm_autotune_noalloc": (ctypes.c_int, [ctypes.POINTER(tg_gemm_args), ctypes.c_int,
                                                ctypes.POINTER(tg_autotune_entry), ctypes.c_void_p]),
    "tg_autotune_cache_size": (ctypes.c_int, []),
    "tg_autotune_cache_get": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(tg_autotune_entry)]),
    "tg_autotune_cache_clear": (ctypes.c_int, []),
    "tg_autotune_cache_save": (ctypes.c_int, [ctypes.c_char_p]),
    "tg_autotune_cache_load": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int),
                                              ctypes.POINTER(ctypes.c_int)]),
    "tg_clock_probe": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "tg_layout_probe": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]),
    "tg_num_configs": (ctypes.c_int, []),
    "tg_get_config": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(tg_tile_config)]),
    "tg_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "tg_version": (ctypes.c_int, []),
}

_lib = None


class TgError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {tg_status_string(status)} ({status})" if what else tg_status_string(status))


def load(build_if_missing: bool = True):
    """Load libtg.so (building it first only if no library exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        if not build_if_missing:
            raise ImportError(f"{LIB_PATH} is missing: run python -m dense_gemm_epilogues_tiled_amd.build")
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


# ---- one-to-one wrappers of the C entry points ------------------------------

def tg_gemm(A: int, B: int, bias: int | None, C: int, M: int, N: int, K: int, dtype: int, epilogue: int,
            stream: int | None) -> int:
    return load().tg_gemm(A, B, bias, C, M, N, K, dtype, epilogue, stream)


def tg_gemm_ex(args: tg_gemm_args, stream: int | None) -> int:
    return load().tg_gemm_ex(ctypes.byref(args), stream)


def tg_gemm_query_config(M: int, N: int, K: int, dtype: int, epilogue: int, b_col_major: int):
    """Returns (status, tg_tile_config)."""
    out = tg_tile_config()
    rc = load().tg_gemm_query_config(M, N, K, dtype, epilogue, b_col_major, ctypes.byref(out))
    return rc, out


def tg_vector_add(A: int | None, B: int | None, C: int | None, n: int, dtype: int, stream: int | None) -> int:
    return load().tg_vector_add(A, B, C, n, dtype, stream)


def tg_row_softmax(X: int | None, Y: int | None, rows: int, cols: int, dtype: int, alpha: float,
                   stream: int | None) -> int:
    return load().tg_row_softmax(X, Y, rows, cols, dtype, alpha, stream)


def tg_attention_fwd(Q: int | None, K: int | None, V: int | None, O: int | None, batch: int, heads: int,
                     seq_len: int, head_dim: int, dtype: int, causal: int, scale: float, stream: int | None) -> int:
    return load().tg_attention_fwd(Q, K, V, O, batch, heads, seq_len, head_dim, dtype, causal, scale, stream)


def tg_gemm_autotune_workspace_size(M: int, N: int, epilogue: int):
    """Returns (status, bytes)."""
    out = ctypes.c_int64(0)
    rc = load().tg_gemm_autotune_workspace_size(M, N, epilogue, ctypes.byref(out))
    return rc, out.value


def tg_gemm_autotune(args: tg_gemm_args | None, workspace: int | None, workspace_bytes: int, iters: int,
                     stream: int | None):
    """Returns (status, tg_autotune_entry)."""
    res = tg_autotune_entry()
    rc = load().tg_gemm_autotune(ctypes.byref(args) if args is not None else None, workspace, workspace_bytes, iters,
                                 ctypes.byref(res), stream)
    return rc, res


def tg_autotune_cache_size() -> int:
    return load().tg_autotune_cache_size()


def tg_autotune_cache_get(index: int):
    """Returns (status, tg_autotune_entry)."""
    out = tg_autotune_entry()
    rc = load().tg_autotune_cache_get(index, ctypes.byref(out))
    return rc, out


def tg_autotune_cache_clear() -> int:
    return load().tg_autotune_cache_clear()


def tg_autotune_cache_save(path: str | None) -> int:
    return load().tg_autotune_cache_save(path.encode() if path is not None else None)


def tg_autotune_cache_load(path: str | None):
    """Returns (status, loaded, skipped)."""
    a, b = ctypes.c_int(0), ctypes.c_int(0)
    rc = load().tg_autotune_cache_load(path.encode() if path is not None else None, ctypes.byref(a), ctypes.byref(b))
    return rc, a.value, b.value


def tg_clock_probe(out: int | None, blocks: int, iters: int, stream: int | None) -> int:
    return load().tg_clock_probe(out, blocks, iters, stream)


def tg_num_configs() -> int:
    return load().tg_num_configs()


def tg_get_config(index: int):
    """Returns (status, tg_tile_config)."""
    out = tg_tile_config()
    rc = load().tg_get_config(index, ctypes.byref(out))
    return rc, out


def tg_status_string(status: int) -> str:
    return load().tg_status_string(status).decode()


def tg_version() -> int:
    return load().tg_version()


# ---- tensor-level helper -----------------------------------------------------

def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def gemm(A: torch.Tensor, B: torch.Tensor, bias: torch.Tensor | None = None, epilogue: str = "none",
         b_col_major: bool = False, alpha: float = 1.0, out: torch.Tensor | None = None, config_id: int = -1,
         stream: int | None = None, group_m: int = 0, xcd_remap: int = -1) -> torch.Tensor:
    """C = epilogue(alpha * A @ B + bias) on the GPU through tg_gemm_ex.

    A: (M, K); B: (K, N), or (N, K) when b_col_major; bias: (N,) for the bias
    epilogues.  fp16 or bf16, contiguous, on one HIP device.  The result has
    the input dtype, or fp32 for ``epilogue="softmax"``.
    """
    if epilogue not in EPILOGUES:
        raise ValueError(f"unknown epilogue {epilogue!r}")
    epi = EPILOGUES[epilogue]
    if A.dtype not in DTYPES or B.dtype != A.dtype or (bias is not None and bias.dtype != A.dtype):
        raise TypeError("A, B and bias must share one dtype, float16 or bfloat16")
    if not (A.is_cuda and B.is_cuda and (bias is None or bias.is_cuda)):
        raise ValueError("tensors must be on a GPU")
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    M, K = A.shape
    if b_col_major:
        N, Kb = B.shape
    else:
        Kb, N = B.shape
    if Kb != K:
        raise ValueError(f"inner dimensions differ: A is {tuple(A.shape)}, B is {tuple(B.shape)}")
    if bias is not None and (bias.dim() != 1 or bias.shape[0] != N):
        raise ValueError("bias must have shape (N,)")
    for name, t in (("A", A), ("B", B), ("bias", bias)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    out_dtype = torch.float32 if epi == TG_EPI_SOFTMAX else A.dtype
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A.device)
    elif out.shape != (M, N) or out.dtype != out_dtype or not out.is_contiguous() or out.device != A.device:
        raise ValueError("out has the wrong shape, dtype, layout or device")
    args = tg_gemm_args(A.data_ptr(), B.data_ptr(), bias.data_ptr() if bias is not None else None, out.data_ptr(),
                        M, N, K, DTYPES[A.dtype], epi, int(bool(b_col_major)), float(alpha), int(config_id),
                        int(group_m), int(xcd_remap))
    rc = tg_gemm_ex(args, stream if stream is not None else _stream_handle(A.device))
    if rc != TG_OK:
        raise TgError(rc, "tg_gemm_ex")
    return out


def vector_add(A: torch.Tensor, B: torch.Tensor, out: torch.Tensor | None = None,
               stream: int | None = None) -> torch.Tensor:
    """C = A + B elementwise on the GPU through tg_vector_add (fp16, bf16 or fp32,
    contiguous, same shape and dtype; ``out`` may be A or B)."""
    if A.dtype not in STREAM_DTYPES or B.dtype != A.dtype:
        raise TypeError("A and B must share one dtype: float16, bfloat16 or float32")
    if not (A.is_cuda and B.is_cuda) or A.device != B.device:
        raise ValueError("tensors must be on one GPU")
    if A.shape != B.shape or not A.is_contiguous() or not B.is_contiguous():
        raise ValueError("A and B must be contiguous and of one shape")
    if out is None:
        out = torch.empty_like(A)
    elif out.shape != A.shape or out.dtype != A.dtype or not out.is_contiguous() or out.device != A.device:
        raise ValueError("out has the wrong shape, dtype, layout or device")
    rc = tg_vector_add(A.data_ptr(), B.data_ptr(), out.data_ptr(), A.numel(), STREAM_DTYPES[A.dtype],
                       stream if stream is not None else _stream_handle(A.device))
    if rc != TG_OK:
        raise TgError(rc, "tg_vector_add")
    return out


def row_softmax(X: torch.Tensor, alpha: float = 1.0, out: torch.Tensor | None = None,
                stream: int | None = None) -> torch.Tensor:
    """Y = softmax(alpha * X) along the last dimension of a contiguous 2-D X
    (fp16, bf16 or fp32) through tg_row_softmax; Y is fp32."""
    if X.dtype not in STREAM_DTYPES:
        raise TypeError("X must be float16, bfloat16 or float32")
    if not X.is_cuda or X.dim() != 2 or not X.is_contiguous():
        raise ValueError("X must be a contiguous 2-D GPU tensor")
    rows, cols = X.shape
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=X.device)
    elif out.shape != X.shape or out.dtype != torch.float32 or not out.is_contiguous() or out.device != X.device:
        raise ValueError("out has the wrong shape, dtype, layout or device")
    rc = tg_row_softmax(X.data_ptr(), out.data_ptr(), rows, cols, STREAM_DTYPES[X.dtype], float(alpha),
                        stream if stream is not None else _stream_handle(X.device))
    if rc != TG_OK:
        raise TgError(rc, "tg_row_softmax")
    return out


def attention(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, causal: bool = False, scale: float | None = None,
              out: torch.Tensor | None = None, stream: int | None = None) -> torch.Tensor:
    """FlashAttention forward through tg_attention_fwd: O = softmax(scale Q K^T [causal]) V.

    Q, K, V: (batch, heads, seq_len, head_dim) contiguous fp16 or bf16 on one GPU
    (head_dim 64 or 128); scale defaults to 1/sqrt(head_dim).  O has Q's shape and dtype.
    """
    if Q.dtype not in DTYPES or K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise TypeError("Q, K and V must share one dtype, float16 or bfloat16")
    if not (Q.is_cuda and K.is_cuda and V.is_cuda) or not (Q.device == K.device == V.device):
        raise ValueError("Q, K and V must be on one GPU")
    if Q.dim() != 4 or K.shape != Q.shape or V.shape != Q.shape:
        raise ValueError("Q, K and V must be 4-D (batch, heads, seq_len, head_dim) of one shape")
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, H, N, D = Q.shape
    if out is None:
        out = torch.empty_like(Q)
    elif out.shape != Q.shape or out.dtype != Q.dtype or not out.is_contiguous() or out.device != Q.device:
        raise ValueError("out has the wrong shape, dtype, layout or device")
    sc = float(D) ** -0.5 if scale is None else float(scale)
    rc = tg_attention_fwd(Q.data_ptr(), K.data_ptr(), V.data_ptr(), out.data_ptr(), B, H, N, D, DTYPES[Q.dtype],
                          int(bool(causal)), sc, stream if stream is not None else _stream_handle(Q.device))
    if rc != TG_OK:
        raise TgError(rc, "tg_attention_fwd")
    return out


def tg_layout_probe(kind: int, out: int | None, stream: int | None) -> int:
    return load().tg_layout_probe(kind, out, stream)


def tg_gemm_autotune_noalloc(args: tg_gemm_args | None, iters: int, stream: int | None):
    """Returns (status, tg_autotune_entry)."""
    res = tg_autotune_entry()
    rc = load().tg_gemm_autotune_noalloc(ctypes.byref(args) if args is not None else None, iters, ctypes.byref(res),
                                         stream)
    return rc, res


def autotune(A: torch.Tensor, B: torch.Tensor, bias: torch.Tensor | None = None, epilogue: str = "none",
             b_col_major: bool = False, alpha: float = 1.0, out: torch.Tensor | None = None, iters: int = 10,
             stream: int | None = None) -> dict:
    """Tune the configuration for this problem (tg_gemm_autotune) and cache it;
    `out` (allocated if None) receives the winner's result.  Returns the cache
    entry as a dict (config, us, candidates, valid) plus "out"."""
    if epilogue not in EPILOGUES:
        raise ValueError(f"unknown epilogue {epilogue!r}")
    epi = EPILOGUES[epilogue]
    if A.dtype not in DTYPES or B.dtype != A.dtype or not (A.is_cuda and B.is_cuda):
        raise ValueError("A and B must be fp16 / bf16 GPU tensors of one dtype")
    M, K = A.shape
    N = B.shape[0] if b_col_major else B.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32 if epi == TG_EPI_SOFTMAX else A.dtype, device=A.device)
    rc, need = tg_gemm_autotune_workspace_size(M, N, epi)
    if rc != TG_OK:
        raise TgError(rc, "tg_gemm_autotune_workspace_size")
    ws = torch.empty(need + 256, dtype=torch.uint8, device=A.device)
    base = (ws.data_ptr() + 255) // 256 * 256
    args = tg_gemm_args(A.data_ptr(), B.data_ptr(), bias.data_ptr() if bias is not None else None, out.data_ptr(),
                        M, N, K, DTYPES[A.dtype], epi, int(bool(b_col_major)), float(alpha), -1, 0, -1)
    rc, res = tg_gemm_autotune(args, base, need, int(iters), stream if stream is not None else _stream_handle(A.device))
    if rc != TG_OK:
        raise TgError(rc, "tg_gemm_autotune")
    d = res.as_dict()
    d["out"] = out
    return d


def autotune_cache() -> list[dict]:
    out = []
    for i in range(tg_autotune_cache_size()):
        rc, e = tg_autotune_cache_get(i)
        if rc != TG_OK:
            raise TgError(rc, "tg_autotune_cache_get")
        out.append(e.as_dict())
    return out


def shader_clock_mhz(device=None, blocks: int = 1024, iters: int = 300000) -> dict:
    """The shader clock under sustained MFMA load, from tg_clock_probe: median
    over workgroups of 100 MHz x shader cycles / constant-counter ticks.  Also
    returns the constant counter's rate against the host clock (should be
    ~100 MHz) and the dense fp16 MFMA peak at the measured clock."""
    import time as _time
    dev = torch.device(device if device is not None else "cuda:0")
    out = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
    torch.cuda.synchronize(dev)
    t0 = _time.perf_counter()
    rc = tg_clock_probe(out.data_ptr(), blocks, iters, _stream_handle(dev))
    if rc != TG_OK:
        raise TgError(rc, "tg_clock_probe")
    torch.cuda.synchronize(dev)
    wall = _time.perf_counter() - t0
    v = out.view(blocks, 2).cpu().double()
    mhz = float((100.0 * v[:, 0] / v[:, 1]).median())
    tick_rate = float(v[:, 1].max()) / wall / 1e6 if wall > 0 else float("nan")  # MHz, lower bound
    return {"mhz": mhz, "realtime_mhz_vs_host": tick_rate, "blocks": blocks, "iters": iters,
            "peak_tflops_at_clock": 256 * 4096 * mhz * 1e6 / 1e12}


def query_config(M: int, N: int, K: int, dtype: torch.dtype, epilogue: str, b_col_major: bool = False) -> dict:
    rc, cfg = tg_gemm_query_config(M, N, K, DTYPES[dtype], EPILOGUES[epilogue], int(bool(b_col_major)))
    if rc != TG_OK:
        raise TgError(rc, "tg_gemm_query_config")
    return cfg.as_dict()


def configs() -> list[dict]:
    out = []
    for i in range(tg_num_configs()):
        rc, cfg = tg_get_config(i)
        if rc != TG_OK:
            raise TgError(rc, "tg_get_config")
        out.append(cfg.as_dict())
    return out
