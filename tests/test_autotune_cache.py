"""The run-time autotune cache without a GPU: file loading and its checks,
save round trip, lookup precedence over the built-in table, clearing, and the
autotuner's argument errors (all raised before any HIP call)."""

import os

import pytest

import dense_gemm_epilogues_tiled_amd as tg

HEADER = "tg-autotune-cache 1\n"


@pytest.fixture(autouse=True)
def _clean_cache():
    tg.tg_autotune_cache_clear()
    yield
    tg.tg_autotune_cache_clear()


def _gemm_cfg(i=0):
    return [c for c in tg.configs() if c["kind"] == tg.TG_KERNEL_GEMM][i]


def _line(c, dtype=0, bcol=0, kind=None, M=1024, N=1024, K=1024, gm=3, xcd=1, us=12.5, **over):
    f = dict(id=c["id"], bm=c["bm"], bn=c["bn"], bk=c["bk"], stages=c["stages"], waves=c["waves"])
    f.update(over)
    kind = c["kind"] if kind is None else kind
    return (f"{dtype} {bcol} {kind} {M} {N} {K} {f['id']} {f['bm']} {f['bn']} {f['bk']} {f['stages']} {f['waves']} "
            f"{gm} {xcd} {us}\n")


def test_loaded_entry_takes_precedence_over_the_table(tmp_path):
    c = _gemm_cfg(1)
    default = tg.query_config(1024, 1024, 1024, tg.torch.float16, "gelu")
    p = tmp_path / "cache.txt"
    p.write_text(HEADER + _line(c))
    assert tg.tg_autotune_cache_load(str(p)) == (tg.TG_OK, 1, 0)
    assert tg.tg_autotune_cache_size() == 1
    for epi in ("none", "bias", "relu", "gelu"):  # one key for every elementwise epilogue
        q = tg.query_config(1024, 1024, 1024, tg.torch.float16, epi)
        assert (q["id"], q["group_m"], q["xcd_remap"]) == (c["id"], 3, 1)
    # other keys are untouched
    assert tg.query_config(1024, 1024, 1024, tg.torch.bfloat16, "gelu") == \
        tg.query_config(1024, 1024, 1024, tg.torch.bfloat16, "gelu")
    assert tg.query_config(1024, 1024, 1032, tg.torch.float16, "gelu")["id"] == \
        tg.query_config(1024, 1024, 1032, tg.torch.float16, "gelu")["id"]
    e = tg.autotune_cache()[0]
    assert (e["M"], e["N"], e["K"], e["dtype"], e["kind"], e["us"]) == (1024, 1024, 1024, 0, 0, 12.5)
    assert tg.tg_autotune_cache_clear() == tg.TG_OK and tg.tg_autotune_cache_size() == 0
    assert tg.query_config(1024, 1024, 1024, tg.torch.float16, "gelu") == default


def test_stale_or_invalid_entries_are_skipped(tmp_path):
    g = _gemm_cfg(0)
    sm = [c for c in tg.configs() if c["kind"] == tg.TG_KERNEL_GEMM_SOFTMAX]
    small = min(sm, key=lambda c: c["bn"])
    lines = [
        _line(g, bm=g["bm"] * 2),                       # id describes another variant (another build)
        _line(g, id=999),                               # no such id
        _line(g, gm=0),                                 # bad raster band
        _line(g, xcd=2),                                # bad regrouping flag
        _line(g, dtype=2),                              # fp32 GEMM does not exist
        _line(g, K=20),                                 # the library rejects K % 8 != 0
        _line(g, kind=tg.TG_KERNEL_GEMM_SOFTMAX),       # kind does not match the id
        _line(small, N=small["bn"] + 8, bcol=small["b_col_major"] if small["b_col_major"] >= 0 else 0),  # row too long
        "1 2 3\n",                                      # malformed
        _line(g, M=2048),                               # the one good line
    ]
    p = tmp_path / "cache.txt"
    p.write_text(HEADER + "# comment\n\n" + "".join(lines))
    assert tg.tg_autotune_cache_load(str(p)) == (tg.TG_OK, 1, len(lines) - 1)
    assert tg.autotune_cache()[0]["M"] == 2048


def test_bad_files(tmp_path):
    assert tg.tg_autotune_cache_load(str(tmp_path / "missing.txt"))[0] == tg.TG_ERR_INVALID_ARG
    p = tmp_path / "bad.txt"
    p.write_text("not a cache\n" + _line(_gemm_cfg()))
    assert tg.tg_autotune_cache_load(str(p))[0] == tg.TG_ERR_INVALID_ARG
    p.write_text("tg-autotune-cache 2\n")
    assert tg.tg_autotune_cache_load(str(p))[0] == tg.TG_ERR_INVALID_ARG
    assert tg.tg_autotune_cache_load(None)[0] == tg.TG_ERR_INVALID_ARG
    assert tg.tg_autotune_cache_save(None) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_autotune_cache_save(str(tmp_path / "no" / "such" / "dir.txt")) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_autotune_cache_get(0)[0] == tg.TG_ERR_INVALID_ARG
    assert tg.load().tg_autotune_cache_get(0, None) == tg.TG_ERR_INVALID_ARG


def test_save_load_round_trip_and_replacement(tmp_path):
    a, b = _gemm_cfg(0), _gemm_cfg(2)
    p = tmp_path / "in.txt"
    p.write_text(HEADER + _line(a, M=512) + _line(b, M=768, dtype=1, bcol=1, gm=8, xcd=0, us=3.25))
    assert tg.tg_autotune_cache_load(str(p))[1] == 2
    q = tmp_path / "out.txt"
    assert tg.tg_autotune_cache_save(str(q)) == tg.TG_OK
    tg.tg_autotune_cache_clear()
    assert tg.tg_autotune_cache_load(str(q)) == (tg.TG_OK, 2, 0)
    got = sorted((e["M"], e["dtype"], e["b_col_major"], e["config"]["id"], e["config"]["group_m"],
                  e["config"]["xcd_remap"], e["us"]) for e in tg.autotune_cache())
    assert got == [(512, 0, 0, a["id"], 3, 1, 12.5), (768, 1, 1, b["id"], 8, 0, 3.25)]
    # loading the same key again replaces the entry instead of adding one
    p.write_text(HEADER + _line(b, M=512, gm=16))
    assert tg.tg_autotune_cache_load(str(p))[1] == 1
    assert tg.tg_autotune_cache_size() == 2
    e = [e for e in tg.autotune_cache() if e["M"] == 512][0]
    assert (e["config"]["id"], e["config"]["group_m"]) == (b["id"], 16)


def test_workspace_size():
    rc, n = tg.tg_gemm_autotune_workspace_size(100, 64, tg.TG_EPI_BIAS_GELU)
    assert rc == tg.TG_OK and n >= 100 * 64 * 2 + 4096
    rc, n2 = tg.tg_gemm_autotune_workspace_size(100, 64, tg.TG_EPI_SOFTMAX)
    assert rc == tg.TG_OK and n2 >= 100 * 64 * 4 + 4096
    assert tg.tg_gemm_autotune_workspace_size(-1, 64, 0)[0] == tg.TG_ERR_INVALID_ARG
    assert tg.tg_gemm_autotune_workspace_size(1, 64, 9)[0] == tg.TG_ERR_INVALID_ARG
    assert tg.load().tg_gemm_autotune_workspace_size(1, 64, 0, None) == tg.TG_ERR_INVALID_ARG
    # beyond the GEMM's limits the byte count would overflow int64: refused
    assert tg.tg_gemm_autotune_workspace_size((1 << 63) - 1, 1 << 20, 0)[0] == tg.TG_ERR_UNSUPPORTED
    assert tg.tg_gemm_autotune_workspace_size(64, (1 << 24) + 8, tg.TG_EPI_SOFTMAX)[0] == tg.TG_ERR_UNSUPPORTED
    assert tg.tg_gemm_autotune_workspace_size((1 << 31) - 1, 1 << 24, tg.TG_EPI_SOFTMAX) == \
        (tg.TG_OK, (((1 << 31) - 1) * (1 << 24) * 4 + 255) // 256 * 256 + 1024 * 4 + 256)


@pytest.mark.parametrize("change,expect", [
    (dict(args=None), tg.TG_ERR_INVALID_ARG),
    (dict(iters=0), tg.TG_ERR_INVALID_ARG),
    (dict(iters=1001), tg.TG_ERR_INVALID_ARG),
    (dict(M=0), tg.TG_ERR_INVALID_ARG),                 # nothing to time
    (dict(N=12), tg.TG_ERR_MISALIGNED),                 # shape errors of tg_gemm_ex
    (dict(dtype=5), tg.TG_ERR_INVALID_ARG),
    (dict(workspace=None), tg.TG_ERR_INVALID_ARG),
    (dict(ws_bytes=100), tg.TG_ERR_INVALID_ARG),        # too small
    (dict(workspace=1 << 20 | 16), tg.TG_ERR_MISALIGNED),
])
def test_autotune_rejects_before_any_hip_call(change, expect):
    M, N, K, dt = change.get("M", 256), change.get("N", 256), 64, change.get("dtype", 0)
    args = tg.tg_gemm_args(4096, 8192, None, 12288, M, N, K, dt, 0, 0, 1.0, -1, 0, -1)
    need = tg.tg_gemm_autotune_workspace_size(max(M, 0), N, 0)[1]
    rc, _ = tg.tg_gemm_autotune(change.get("args", args), change.get("workspace", 1 << 20),
                                change.get("ws_bytes", need), change.get("iters", 5), None)
    assert rc == expect
    assert tg.tg_autotune_cache_size() == 0
