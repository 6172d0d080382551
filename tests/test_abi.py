"""C-ABI contract of libtg.so, checked without a GPU.

Every symbol include/tg.h declares is exported; every invalid argument is
rejected with its documented status before any HIP call (these calls never
touch a device, so they run on a machine without one); the configuration
query and table are self-consistent.
"""

import ctypes
import os
import re
import subprocess

import pytest

import dense_gemm_epilogues_tiled_amd as tg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tg.h")
_FIRST_SOFTMAX = min(c["id"] for c in tg.configs() if c["kind"] == tg.TG_KERNEL_GEMM_SOFTMAX)


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tg_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    for n in ("tg_gemm", "tg_gemm_ex", "tg_gemm_query_config", "tg_num_configs", "tg_get_config",
              "tg_status_string", "tg_version", "tg_vector_add", "tg_row_softmax", "tg_attention_fwd",
              "tg_gemm_autotune", "tg_gemm_autotune_workspace_size", "tg_autotune_cache_size", "tg_autotune_cache_get",
              "tg_autotune_cache_clear", "tg_autotune_cache_save", "tg_autotune_cache_load", "tg_clock_probe"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(tg.LIB_PATH)
    for n in _declared_functions():
        assert hasattr(lib, n), f"{n} declared in tg.h but not exported"
    assert set(_declared_functions()) == set(tg._SIGNATURES), "binding and header disagree"


def test_struct_layouts_match_header(tmp_path):
    """The ctypes mirrors have the C compiler's sizes and field offsets."""
    fields = {"tg_tile_config": [f for f, _ in tg.tg_tile_config._fields_],
              "tg_gemm_args": [f for f, _ in tg.tg_gemm_args._fields_],
              "tg_autotune_entry": [f for f, _ in tg.tg_autotune_entry._fields_]}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "tg.h"', "int main(void) {"]
    for st, fs in fields.items():
        lines.append(f'  printf("{st} %zu\\n", sizeof({st}));')
        for f in fs:
            lines.append(f'  printf("{st}.{f} %zu\\n", offsetof({st}, {f}));')
    lines.append("  return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                 check=True).stdout.splitlines())
    for st, cls in (("tg_tile_config", tg.tg_tile_config), ("tg_gemm_args", tg.tg_gemm_args),
                    ("tg_autotune_entry", tg.tg_autotune_entry)):
        assert int(got[st]) == ctypes.sizeof(cls)
        for f in fields[st]:
            assert int(got[f"{st}.{f}"]) == getattr(cls, f).offset, f


def test_status_strings():
    for s in (tg.TG_OK, tg.TG_ERR_INVALID_ARG, tg.TG_ERR_UNSUPPORTED, tg.TG_ERR_MISALIGNED, tg.TG_ERR_HIP):
        assert tg.tg_status_string(s).startswith("TG_")
    assert "unknown" in tg.tg_status_string(12345)
    assert tg.tg_version() == 1


def test_config_table():
    n = tg.tg_num_configs()
    assert n >= 4
    kinds = set()
    for i in range(n):
        rc, c = tg.tg_get_config(i)
        assert rc == tg.TG_OK and c.id == i
        kinds.add(c.kind)
        assert c.lds_bytes <= 160 * 1024, "LDS budget of a gfx950 CU"
        # one wave per wave_m x wave_n block, or two that split each K step
        assert c.waves in (c.wave_m * c.wave_n, 2 * c.wave_m * c.wave_n)
        if c.kind == tg.TG_KERNEL_GEMM:
            assert c.bm % (16 * c.wave_m) == 0 and c.bn % (16 * c.wave_n) == 0
    assert kinds == {tg.TG_KERNEL_GEMM, tg.TG_KERNEL_GEMM_SOFTMAX}
    assert tg.tg_get_config(-1)[0] == tg.TG_ERR_INVALID_ARG
    assert tg.tg_get_config(n)[0] == tg.TG_ERR_INVALID_ARG
    assert tg.load().tg_get_config(0, None) == tg.TG_ERR_INVALID_ARG


def test_query_picks_kind_and_layout():
    for epi in ("none", "bias", "relu", "gelu"):
        c = tg.query_config(2048, 2048, 2048, tg.torch.float16, epi)
        assert c["kind"] == tg.TG_KERNEL_GEMM
    c = tg.query_config(4096, 1024, 128, tg.torch.float16, "softmax", True)
    assert c["kind"] == tg.TG_KERNEL_GEMM_SOFTMAX and c["b_col_major"] == 1 and c["bn"] >= 1024
    c = tg.query_config(64, 2048, 64, tg.torch.bfloat16, "softmax")
    assert c["bn"] >= 2048
    # every-CU rule: a big problem gets a big tile, a small one a small tile
    assert tg.query_config(16384, 16384, 1024, tg.torch.bfloat16, "relu")["bm"] == 256
    assert tg.query_config(64, 64, 64, tg.torch.float16, "none")["bm"] * tg.query_config(
        64, 64, 64, tg.torch.float16, "none")["bn"] <= 128 * 128


@pytest.mark.parametrize("args,expect", [
    (dict(M=-1), tg.TG_ERR_INVALID_ARG),
    (dict(N=-8), tg.TG_ERR_INVALID_ARG),
    (dict(K=-8), tg.TG_ERR_INVALID_ARG),
    (dict(dtype=tg.TG_DTYPE_F32), tg.TG_ERR_INVALID_ARG),  # fp32 is for the bandwidth kernels only
    (dict(dtype=7), tg.TG_ERR_INVALID_ARG),
    (dict(epilogue=5), tg.TG_ERR_INVALID_ARG),
    (dict(epilogue=-1), tg.TG_ERR_INVALID_ARG),
    (dict(b_col_major=2), tg.TG_ERR_INVALID_ARG),
    (dict(N=12), tg.TG_ERR_MISALIGNED),
    (dict(K=20), tg.TG_ERR_MISALIGNED),
    (dict(M=1 << 31), tg.TG_ERR_UNSUPPORTED),
    (dict(N=(1 << 24) + 8), tg.TG_ERR_UNSUPPORTED),
    (dict(K=(1 << 20) + 8), tg.TG_ERR_UNSUPPORTED),
    (dict(epilogue=tg.TG_EPI_SOFTMAX, N=tg.TG_SOFTMAX_MAX_N + 8), tg.TG_ERR_UNSUPPORTED),
    (dict(A=0), tg.TG_ERR_INVALID_ARG),
    (dict(B=0), tg.TG_ERR_INVALID_ARG),
    (dict(C=0), tg.TG_ERR_INVALID_ARG),
    (dict(bias=0, epilogue=tg.TG_EPI_BIAS), tg.TG_ERR_INVALID_ARG),       # bias required
    (dict(bias=4096, epilogue=tg.TG_EPI_NONE), tg.TG_ERR_INVALID_ARG),     # bias forbidden
    (dict(bias=4096, epilogue=tg.TG_EPI_SOFTMAX), tg.TG_ERR_INVALID_ARG),  # bias forbidden
    (dict(A=4104), tg.TG_ERR_MISALIGNED),
    (dict(B=4100), tg.TG_ERR_MISALIGNED),
    (dict(C=4098), tg.TG_ERR_MISALIGNED),
    (dict(bias=4104, epilogue=tg.TG_EPI_BIAS_GELU), tg.TG_ERR_MISALIGNED),
    (dict(config_id=99), tg.TG_ERR_INVALID_ARG),
    (dict(config_id=_FIRST_SOFTMAX), tg.TG_ERR_INVALID_ARG),               # softmax config for a GEMM
    (dict(config_id=0, epilogue=tg.TG_EPI_SOFTMAX), tg.TG_ERR_INVALID_ARG),  # GEMM config for softmax
    (dict(config_id=_FIRST_SOFTMAX, epilogue=tg.TG_EPI_SOFTMAX, N=2048), tg.TG_ERR_UNSUPPORTED),  # row too long
    (dict(group_m=-1), tg.TG_ERR_INVALID_ARG),
    (dict(xcd_remap=2), tg.TG_ERR_INVALID_ARG),
])
def test_invalid_arguments_rejected_before_any_hip_call(args, expect):
    # fake, never-dereferenced device addresses: validation must fail first
    base = dict(A=4096, B=8192, bias=None, C=12288, M=64, N=64, K=64, dtype=0, epilogue=0, b_col_major=0,
                alpha=1.0, config_id=-1, group_m=0, xcd_remap=-1)
    base.update(args)
    if base["bias"] == 0:
        base["bias"] = None
    a = tg.tg_gemm_args(base["A"] or None, base["B"] or None, base["bias"], base["C"] or None, base["M"], base["N"],
                        base["K"], base["dtype"], base["epilogue"], base["b_col_major"], base["alpha"],
                        base["config_id"], base["group_m"], base["xcd_remap"])
    assert tg.tg_gemm_ex(a, None) == expect


def test_layout_specific_variant_rejects_other_layout():
    only_col = [c["id"] for c in tg.configs() if c["kind"] == tg.TG_KERNEL_GEMM_SOFTMAX and c["b_col_major"] == 1]
    assert only_col, "a column-major-only softmax variant is compiled"
    a = tg.tg_gemm_args(4096, 8192, None, 12288, 64, 64, 64, 0, tg.TG_EPI_SOFTMAX, 0, 1.0, only_col[0], 0, -1)
    assert tg.tg_gemm_ex(a, None) == tg.TG_ERR_INVALID_ARG


def test_null_args_struct():
    assert tg.load().tg_gemm_ex(None, None) == tg.TG_ERR_INVALID_ARG


def test_empty_problems_launch_nothing():
    # M == 0 or N == 0: TG_OK with no device touched (NULL pointers are fine)
    assert tg.tg_gemm(None, None, None, None, 0, 64, 64, 0, 0, None) == tg.TG_OK
    assert tg.tg_gemm(None, None, None, None, 64, 0, 64, 1, 0, None) == tg.TG_OK
    assert tg.tg_gemm(None, None, None, None, 0, 0, 0, 0, tg.TG_EPI_SOFTMAX, None) == tg.TG_OK


def test_query_rejects_bad_input():
    assert tg.tg_gemm_query_config(-1, 8, 8, 0, 0, 0)[0] == tg.TG_ERR_INVALID_ARG
    assert tg.tg_gemm_query_config(8, 8, 8, 3, 0, 0)[0] == tg.TG_ERR_INVALID_ARG
    assert tg.tg_gemm_query_config(8, 4096, 8, 0, tg.TG_EPI_SOFTMAX, 1)[0] == tg.TG_ERR_UNSUPPORTED
    assert tg.load().tg_gemm_query_config(8, 8, 8, 0, 0, 0, None) == tg.TG_ERR_INVALID_ARG


def test_torch_wrapper_checks_before_launch():
    import torch
    a = torch.zeros(4, 8, dtype=torch.float16)
    with pytest.raises(ValueError):
        tg.gemm(a, a.t().contiguous())  # CPU tensors are refused
    with pytest.raises(TypeError):
        tg.gemm(a.float(), a.float())
    with pytest.raises(ValueError):
        tg.gemm(a, a, epilogue="tanh")


# ---- the two bandwidth-bound entry points --------------------------------------

@pytest.mark.parametrize("args,expect", [
    (dict(n=-1), tg.TG_ERR_INVALID_ARG),
    (dict(n=(1 << 36) + 1), tg.TG_ERR_UNSUPPORTED),
    (dict(dtype=3), tg.TG_ERR_INVALID_ARG),
    (dict(dtype=-1), tg.TG_ERR_INVALID_ARG),
    (dict(A=0), tg.TG_ERR_INVALID_ARG),
    (dict(B=0), tg.TG_ERR_INVALID_ARG),
    (dict(C=0), tg.TG_ERR_INVALID_ARG),
    (dict(A=4100), tg.TG_ERR_MISALIGNED),
    (dict(B=8200), tg.TG_ERR_MISALIGNED),
    (dict(C=12290), tg.TG_ERR_MISALIGNED),
])
def test_vector_add_rejects_before_any_hip_call(args, expect):
    base = dict(A=4096, B=8192, C=12288, n=1000, dtype=tg.TG_DTYPE_F32)
    base.update(args)
    assert tg.tg_vector_add(base["A"] or None, base["B"] or None, base["C"] or None, base["n"], base["dtype"],
                            None) == expect


def test_vector_add_empty_launches_nothing():
    for dt in (tg.TG_DTYPE_F16, tg.TG_DTYPE_BF16, tg.TG_DTYPE_F32):
        assert tg.tg_vector_add(None, None, None, 0, dt, None) == tg.TG_OK
    assert tg.tg_vector_add(None, None, None, 0, 5, None) == tg.TG_ERR_INVALID_ARG  # dtype still checked


@pytest.mark.parametrize("args,expect", [
    (dict(rows=-1), tg.TG_ERR_INVALID_ARG),
    (dict(cols=-8), tg.TG_ERR_INVALID_ARG),
    (dict(dtype=3), tg.TG_ERR_INVALID_ARG),
    (dict(X=0), tg.TG_ERR_INVALID_ARG),
    (dict(Y=0), tg.TG_ERR_INVALID_ARG),
    (dict(X=4104), tg.TG_ERR_MISALIGNED),
    (dict(Y=8196), tg.TG_ERR_MISALIGNED),
    (dict(cols=12), tg.TG_ERR_MISALIGNED),                                  # fp16 rows of 24 bytes
    (dict(cols=6, dtype=tg.TG_DTYPE_F32), tg.TG_ERR_MISALIGNED),            # fp32 rows of 24 bytes
    (dict(cols=8200), tg.TG_ERR_UNSUPPORTED),                               # beyond 16 KiB of fp16
    (dict(cols=4100, dtype=tg.TG_DTYPE_F32), tg.TG_ERR_UNSUPPORTED),        # beyond 16 KiB of fp32
    (dict(rows=1 << 31), tg.TG_ERR_UNSUPPORTED),
    (dict(cols=(1 << 63) - 1), tg.TG_ERR_UNSUPPORTED),                      # row bytes would overflow int64
    (dict(cols=(1 << 62), dtype=tg.TG_DTYPE_F32), tg.TG_ERR_UNSUPPORTED),
])
def test_row_softmax_rejects_before_any_hip_call(args, expect):
    base = dict(X=4096, Y=8192, rows=16, cols=64, dtype=tg.TG_DTYPE_F16, alpha=1.0)
    base.update(args)
    assert tg.tg_row_softmax(base["X"] or None, base["Y"] or None, base["rows"], base["cols"], base["dtype"],
                             base["alpha"], None) == expect


def test_row_softmax_limits_match_header():
    assert tg.TG_ROW_SOFTMAX_MAX_ROW_BYTES == 16384
    src = open(HEADER).read()
    assert re.search(r"#define TG_ROW_SOFTMAX_MAX_ROW_BYTES 16384\b", src)
    assert re.search(r"TG_DTYPE_F32 = 2\b", src) and tg.TG_DTYPE_F32 == 2


def test_row_softmax_empty_launches_nothing():
    assert tg.tg_row_softmax(None, None, 0, 64, tg.TG_DTYPE_F16, 1.0, None) == tg.TG_OK
    assert tg.tg_row_softmax(None, None, 64, 0, tg.TG_DTYPE_F32, 1.0, None) == tg.TG_OK


def test_stream_wrappers_check_before_launch():
    import torch
    a = torch.zeros(16, dtype=torch.float32)
    with pytest.raises(ValueError):
        tg.vector_add(a, a)  # CPU tensors are refused
    with pytest.raises(TypeError):
        tg.vector_add(a.double(), a.double())
    with pytest.raises(ValueError):
        tg.row_softmax(a.reshape(4, 4))
    with pytest.raises(TypeError):
        tg.row_softmax(a.reshape(4, 4).to(torch.int32))


# ---- attention forward -------------------------------------------------------------

@pytest.mark.parametrize("args,expect", [
    (dict(batch=-1), tg.TG_ERR_INVALID_ARG),
    (dict(heads=-2), tg.TG_ERR_INVALID_ARG),
    (dict(seq_len=-5), tg.TG_ERR_INVALID_ARG),
    (dict(head_dim=-128), tg.TG_ERR_INVALID_ARG),
    (dict(dtype=tg.TG_DTYPE_F32), tg.TG_ERR_INVALID_ARG),
    (dict(dtype=9), tg.TG_ERR_INVALID_ARG),
    (dict(causal=2), tg.TG_ERR_INVALID_ARG),
    (dict(scale=float("nan")), tg.TG_ERR_INVALID_ARG),
    (dict(scale=float("inf")), tg.TG_ERR_INVALID_ARG),
    (dict(head_dim=32), tg.TG_ERR_UNSUPPORTED),
    (dict(head_dim=96), tg.TG_ERR_UNSUPPORTED),
    (dict(head_dim=256), tg.TG_ERR_UNSUPPORTED),
    (dict(head_dim=1 << 40), tg.TG_ERR_UNSUPPORTED),
    (dict(seq_len=(1 << 20) + 1), tg.TG_ERR_UNSUPPORTED),
    (dict(batch=1 << 20, heads=1 << 12), tg.TG_ERR_UNSUPPORTED),   # grid of 2^32 workgroups
    (dict(batch=1 << 62, heads=4), tg.TG_ERR_UNSUPPORTED),          # product would overflow
    (dict(Q=0), tg.TG_ERR_INVALID_ARG),
    (dict(K=0), tg.TG_ERR_INVALID_ARG),
    (dict(V=0), tg.TG_ERR_INVALID_ARG),
    (dict(O=0), tg.TG_ERR_INVALID_ARG),
    (dict(Q=4104), tg.TG_ERR_MISALIGNED),
    (dict(K=8200), tg.TG_ERR_MISALIGNED),
    (dict(V=12290), tg.TG_ERR_MISALIGNED),
    (dict(O=16392), tg.TG_ERR_MISALIGNED),
])
def test_attention_rejects_before_any_hip_call(args, expect):
    base = dict(Q=4096, K=8192, V=12288, O=16384, batch=2, heads=4, seq_len=256, head_dim=128,
                dtype=tg.TG_DTYPE_F16, causal=0, scale=0.125)
    base.update(args)
    assert tg.tg_attention_fwd(base["Q"] or None, base["K"] or None, base["V"] or None, base["O"] or None,
                               base["batch"], base["heads"], base["seq_len"], base["head_dim"], base["dtype"],
                               base["causal"], base["scale"], None) == expect


def test_attention_empty_launches_nothing():
    for b, h, n in ((0, 4, 256), (2, 0, 256), (2, 4, 0)):
        assert tg.tg_attention_fwd(None, None, None, None, b, h, n, 128, tg.TG_DTYPE_BF16, 1, 0.1, None) == tg.TG_OK


def test_attention_wrapper_checks_before_launch():
    import torch
    q = torch.zeros(1, 2, 8, 128, dtype=torch.float16)
    with pytest.raises(ValueError):
        tg.attention(q, q, q)  # CPU tensors are refused
    with pytest.raises(TypeError):
        tg.attention(q.float(), q.float(), q.float())


def test_clock_probe_rejects_before_any_hip_call():
    assert tg.tg_clock_probe(None, 4, 10, None) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_clock_probe(4096, 0, 10, None) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_clock_probe(4096, 65537, 10, None) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_clock_probe(4096, 4, 0, None) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_clock_probe(4096, 4, (1 << 24) + 1, None) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_clock_probe(4100, 4, 10, None) == tg.TG_ERR_MISALIGNED
