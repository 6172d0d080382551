"""GPU: the entry points inside a captured HIP graph.

bench.py times every kernel by replaying a captured graph, so each launch
path is captured here once and replayed several times, with eager work of
the program between the replays (other launches that overwrite the same
output buffers and the inputs of the next replay's reference), and every
replay's output is compared bitwise with an eager launch on the same inputs.
None of the library's launch paths records a memset or a host call, so a
captured launch is the kernel launch alone.
"""

import pytest
import torch

import workloads

tg = pytest.importorskip("dense_gemm_epilogues_tiled_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 4


def _check_replays(launch, out, scramble):
    """Eager result, then capture; per replay: scramble the output eagerly,
    replay, synchronize, compare bitwise with the eager result."""
    stream = torch.cuda.Stream(device=DEV)
    with torch.cuda.stream(stream):
        launch()
    torch.cuda.synchronize()
    want = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        launch()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        scramble(r)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if out.element_size() == 2 else out.view(torch.int32),
                           want.view(torch.int16) if want.element_size() == 2 else want.view(torch.int32)), \
            f"replay {r} differs from the eager result"


@pytest.mark.parametrize("name", ["C3", "C5", "C4b"])
def test_gemm_replays_match_eager(name):
    w = workloads.WORKLOADS[name]
    A, B, bias = workloads.make_inputs(w)
    Ad, Bd = A.to(DEV), B.to(DEV)
    bd = bias.to(DEV) if bias is not None else None
    C = torch.empty((w.M, w.N), dtype=torch.float32 if w.epilogue == "softmax" else Ad.dtype, device=DEV)
    print(f"[graph] {name}: {w.description}", flush=True)

    def launch():
        tg.gemm(Ad, Bd, bd, epilogue=w.epilogue, b_col_major=w.b_col_major, alpha=w.alpha, out=C)

    def scramble(r):
        C.fill_(float(r + 1))
        # another GEMM on the same stream and output in between
        tg.gemm(Ad, Bd, bd, epilogue=w.epilogue, b_col_major=w.b_col_major, alpha=w.alpha * 0.5, out=C)

    _check_replays(launch, C, scramble)


def test_stream_kernels_replay_match_eager():
    a = workloads.random_matrix((1 << 20,), 9201, "f16")
    b = workloads.random_matrix((1 << 20,), 9202, "f16")
    ad, bd = a.to(DEV), b.to(DEV)
    c = torch.empty_like(ad)
    print("[graph] vector add 2^20 fp16", flush=True)
    _check_replays(lambda: tg.vector_add(ad, bd, out=c), c, lambda r: c.fill_(float(r)))

    x = workloads.random_matrix((512, 2048), 9203, "bf16").to(DEV)
    y = torch.empty((512, 2048), dtype=torch.float32, device=DEV)
    print("[graph] row softmax 512 x 2048 bf16", flush=True)
    _check_replays(lambda: tg.row_softmax(x, alpha=0.7, out=y), y, lambda r: y.fill_(-1.0 - r))


@pytest.mark.parametrize("causal", [False, True], ids=["non_causal", "causal"])
def test_attention_replays_match_eager(causal):
    shape = (1, 4, 1024, 128)
    q, k, v = (workloads.random_matrix(shape, 9210 + i + 3 * int(causal), "f16").to(DEV) for i in range(3))
    o = torch.empty_like(q)
    print(f"[graph] attention 1x4x1024x128 fp16 causal={causal}", flush=True)

    def scramble(r):
        o.fill_(float(r))
        tg.attention(q, v, k, causal=causal, out=o)  # K and V swapped: a different result in o

    _check_replays(lambda: tg.attention(q, k, v, causal=causal, out=o), o, scramble)
