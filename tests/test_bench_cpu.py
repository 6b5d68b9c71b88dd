"""Host-side checks of the benchmark's bookkeeping (no GPU needed).

The benchmark's contract is to time exactly --steps calls after exactly
--warmup untimed ones, and to report a roofline `traffic` only for the kernel
sources the committed counter summary was taken on.
"""

import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

import bench  # noqa: E402


class _FakeGraph:
    """Stands in for a captured graph: remembers the call indices captured."""

    def __init__(self, calls):
        self.calls = calls


def _fake_capture(torch, stream, fn, count):
    seen = []
    for i in range(count):
        seen.append(fn(i))
    return _FakeGraph(seen)


@pytest.mark.parametrize("calls", [1, 5, 20, 2047, 2048, 2049, 4096, 5000, 10241])
def test_exact_graphs_make_exactly_the_requested_calls(monkeypatch, calls):
    monkeypatch.setattr(bench, "capture", _fake_capture)
    graphs = bench.exact_graphs(None, None, lambda i: i, calls)
    replayed = []
    for graph, replays in graphs:
        assert replays >= 1
        for _ in range(replays):
            replayed.extend(graph.calls)
    assert len(replayed) == calls
    # One graph of `chunk` calls replayed `full` times repeats its indices;
    # the remainder graph continues after them.
    chunk = 2048
    full, rest = divmod(calls, chunk)
    expect = list(range(chunk)) * full + [full * chunk + i for i in range(rest)]
    assert replayed == expect


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_is_read_for_the_measured_sources_only(tmp_path, monkeypatch):
    # The committed summary carries a line per kernel; each value is returned
    # only while the kernel source and its headers hash to the recorded digest.
    for key, src in (("gemv_traffic_bytes_per_launch", "gemv_tq2_g128_amd/csrc/tq2_gemv.hip"),
                     ("gemv_batched_traffic_bytes_per_launch", "gemv_tq2_g128_amd/csrc/tq2_gemv.hip"),
                     ("gemm_traffic_bytes_per_launch", "gemv_tq2_g128_amd/csrc/tq2_gemm.hip")):
        v = bench.measured_traffic(key, src)
        digest = bench.kernel_source_digest(src)
        with open(os.path.join(ROOT, "profiles", "gemv_k4096_n4096_traffic.md")) as f:
            line = [l for l in f.read().splitlines() if l.startswith("machine-readable: %s=" % key)]
        assert len(line) == 1
        recorded = dict(kv.split("=", 1) for kv in line[0][len("machine-readable: "):].split())
        if recorded["kernel_source_sha256"] == digest:
            assert v == int(recorded[key]) and v > 0
        else:
            assert v is None
    assert bench.measured_traffic("no_such_kernel_traffic_bytes_per_launch",
                                  "gemv_tq2_g128_amd/csrc/tq2_gemv.hip") is None

    # A changed source (here: a copy of the tree with one byte more) gives None.
    fake_root = tmp_path / "repo"
    (fake_root / "gemv_tq2_g128_amd" / "csrc").mkdir(parents=True)
    (fake_root / "profiles").mkdir()
    for rel in ("gemv_tq2_g128_amd/csrc/tq2_gemv.hip",) + bench.KERNEL_HEADERS + (
            "profiles/gemv_k4096_n4096_traffic.md",):
        with open(os.path.join(ROOT, rel), "rb") as f:
            data = f.read()
        if rel.endswith("tq2_gemv.hip"):
            data += b"\n"
        (fake_root / rel).write_bytes(data)
    monkeypatch.setattr(bench.os.path, "abspath", lambda p, _root=str(fake_root / "bench.py"): _root)
    assert bench.measured_traffic("gemv_traffic_bytes_per_launch",
                                  "gemv_tq2_g128_amd/csrc/tq2_gemv.hip") is None
