"""Host-side behaviour of bench.py (no GPU): it refuses more than one GPU with
a message and exit status 2, names the kernel a tile configuration launches
the way the kernel trace does, warms the GPU by wall time before the timed
replay, and labels a bandwidth figure whose working set fits the MALL as
such."""

import contextlib
import os
import subprocess
import sys
import time

import pytest

import dense_gemm_epilogues_tiled_amd as tg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)


def test_kernel_names_follow_the_configuration():
    names = {}
    for c in tg.configs():
        names[c["id"]] = bench.kernel_name(c)
        if c["kind"] == tg.TG_KERNEL_GEMM_SOFTMAX:
            assert names[c["id"]] in ("gemm_softmax_kernel", "gemm_softmax_lds_kernel")
        elif c["waves"] == 2 * c["wave_m"] * c["wave_n"]:
            assert names[c["id"]] == "gemm_ksplit_kernel"
        else:
            assert c["waves"] == c["wave_m"] * c["wave_n"] and names[c["id"]] == "gemm_tile_kernel"
    assert "gemm_ksplit_kernel" in names.values() and "gemm_tile_kernel" in names.values()


class _FakeCuda:
    """Stand-in for torch.cuda that logs the order of calls (no GPU)."""

    def __init__(self, log, launch_s):
        self.log, self.launch_s = log, launch_s
        fake = self

        class Graph:
            def __init__(self):
                self.n = 0

            def replay(self):
                fake.log.append(("replay", self.n))
                time.sleep(fake.launch_s * self.n)

        class Event:
            def __init__(self, enable_timing=False):
                pass

            def record(self, stream=None):
                fake.log.append(("event",))

            def elapsed_time(self, other):
                return 1.0

        self.CUDAGraph, self.Event = Graph, Event
        self._capturing = None

    def synchronize(self):
        self.log.append(("sync",))

    @contextlib.contextmanager
    def stream(self, s):
        yield

    @contextlib.contextmanager
    def graph(self, g, stream=None):
        self._capturing = g
        yield
        self._capturing = None


class _FakeTorch:
    def __init__(self, log, launch_s):
        self.cuda = _FakeCuda(log, launch_s)


def test_headline_warms_up_by_wall_time_before_the_timed_replay():
    # the default the driver's command line gets: at least one second
    assert bench.build_parser().parse_args([]).warm_s >= 1.0
    log = []
    ft = _FakeTorch(log, launch_s=1e-4)

    def launch():
        if ft.cuda._capturing is not None:
            ft.cuda._capturing.n += 1
        else:
            log.append(("eager",))

    wall, ev, warm = bench.time_launches(launch, steps=20, warmup=5, stream=None, warm_s=0.2, torch_mod=ft)
    assert warm >= 0.2
    assert log[:5] == [("eager",)] * 5
    # the warm-up replays the captured 20-launch graph; the timed replay sits
    # between two events after the warm-up
    replays = [i for i, e in enumerate(log) if e[0] == "replay"]
    assert len(replays) >= 2 and all(log[i] == ("replay", 20) for i in replays)
    events = [i for i, e in enumerate(log) if e[0] == "event"]
    assert len(events) == 2 and events[0] < replays[-1] < events[1]
    assert all(i < events[0] for i in replays[:-1])
    assert ev == 1.0 / 20


def test_warm_by_wall_time_runs_at_least_one_batch():
    calls = []
    n, spent = bench.warm_by_wall_time(lambda: calls.append(1), lambda: None, 0.0, batch=3)
    assert n == 3 and len(calls) == 3 and spent >= 0.0


def test_mall_resident_bandwidth_is_labelled():
    import workloads
    # the 4 Mi-element vector add moves 48 MiB: served from the 256 MB MALL
    v1 = workloads.STREAM_WORKLOADS["V1"].min_bytes()
    f = bench.bandwidth_fields(v1, 7000.0)
    assert f["memory_level"] == "mall" and "pct_hbm_peak" not in f
    assert f["pct_hbm_peak_mall_resident"] == pytest.approx(87.5)
    # the 256 Mi-element one moves 3 GiB: an HBM rate
    v2 = workloads.STREAM_WORKLOADS["V2"].min_bytes()
    f = bench.bandwidth_fields(v2, 6000.0)
    assert f["memory_level"] == "hbm" and f["pct_hbm_peak"] == pytest.approx(75.0)
    assert bench.bandwidth_fields(workloads.STREAM_WORKLOADS["S1"].min_bytes(), 1.0)["memory_level"] == "hbm"
