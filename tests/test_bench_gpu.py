"""The benchmark's timing events on the GPU.

bench.TimingEvent records HIP events created with hipEventDisableSystemFence
on the stream the kernels run on.  Over the same region of graph-replayed GEMV
calls it must agree with torch's own events (which add the system-scope fence
to each record) to within that fence's cost.
"""

import os
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))


@pytest.mark.gpu
def test_timing_events_agree_with_torch_events():
    import torch
    import bench
    import tq2_inputs as G
    from gemv_tq2_g128_amd import tq2

    dev = torch.device("cuda:0")
    case = G.config2(with_residual=True)
    n, k = case["n"], case["k"]
    soa = tq2.reformat_aos_to_soa(torch.from_numpy(case["aos"]).to(dev), n, k)
    x = torch.from_numpy(case["x"]).to(dev).reshape(-1)
    res = torch.from_numpy(case["residual"]).to(dev).reshape(-1)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream(dev)

    def call(i):
        st = tq2.gemv_ptr(soa.data_ptr(), x.data_ptr(), res.data_ptr(), out.data_ptr(), n, k,
                          torch.cuda.current_stream(dev).cuda_stream)
        assert st == 0, tq2.status_string(st)

    graph = bench.capture(torch, stream, call, 256)
    hip_ms, torch_ms = [], []
    for _ in range(5):
        for kind, sink in (("hip", hip_ms), ("torch", torch_ms)):
            if kind == "hip":
                a, b = bench.TimingEvent(), bench.TimingEvent()
            else:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                graph.replay()                    # keep the stream busy ahead of the region
                a.record(stream)
                graph.replay()
                b.record(stream)
            torch.cuda.synchronize()
            sink.append(a.elapsed_time(b))
    h, t = min(hip_ms), min(torch_ms)
    assert h > 0.0 and t > 0.0
    # 256 GEMV calls take several hundred microseconds; the two kinds of event
    # differ by the fence (about a microsecond per region) and run-to-run noise.
    assert abs(h - t) <= 0.05 * t + 0.005, (hip_ms, torch_ms)
    # The result of the timed calls is the GEMV's (the events do not disturb it).
    ref = tq2.gemv(soa, x, n, k, residual=res)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
