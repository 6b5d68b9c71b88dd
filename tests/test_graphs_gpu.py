"""Entry points captured into a HIP graph replay the eager results exactly.

The benchmark times every entry point from captured graphs, so captured
launches must compute what eager ones do on every replay.  Each replay here
follows eager work of the program's own (the outputs filled with NaN, other
library calls on other buffers, a synchronisation), and every output of
every replay must equal the eager result bit for bit (the kernels are
deterministic: a fixed reduction order per output).
"""

import numpy as np
import pytest

import tq2_inputs as G

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tq2():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    from gemv_tq2_g128_amd import tq2 as mod
    return mod


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_graph_replays_match_eager(tq2):
    n, k = 1000, 1152
    c = G.random_case(8100, 40, n, k, residual=True)
    soa = tq2.reformat_aos_to_soa(_dev(c["aos"]), n, k)
    q1c = G.random_case_q1(8101, 9, n, k, residual=True)
    soa_q1 = tq2.reformat_aos_to_soa(_dev(q1c["aos"]), n, k, fmt="q1")
    x = _dev(c["x"])
    res = _dev(c["residual"])
    xq = _dev(q1c["x"])
    outs = {
        "gemv": torch.empty(n, device="cuda"),
        "batched": torch.empty(3, n, device="cuda"),
        "skinny": torch.empty(8, n, device="cuda"),
        "tile": torch.empty(40, n, device="cuda"),
        "tile_plain": torch.empty(40, n, device="cuda"),
        "precise": torch.empty(40, n, device="cuda"),
        "swiglu1": torch.empty(1, n, device="cuda"),
        "swiglu40": torch.empty(40, n, device="cuda"),
        "q1gemv": torch.empty(n, device="cuda"),
        "q1gemm": torch.empty(9, n, device="cuda"),
    }

    def calls():
        o = outs
        tq2.gemv(soa, x[0], n, k, residual=res[0], out=o["gemv"])
        tq2.gemv_batched([dict(soa=soa, x=x[i], n=n, k=k, residual=res[i] if i != 1 else None,
                               out=o["batched"][i]) for i in range(3)])
        tq2.gemm(soa, x[:8], n, k, residual=res[:8], out=o["skinny"])
        tq2.gemm(soa, x, n, k, residual=res, out=o["tile"])            # tq2_gemm_ws
        tq2.gemm(soa, x, n, k, residual=res, out=o["tile_plain"], workspace=None)
        tq2.gemm(soa, x, n, k, residual=res, out=o["precise"], precise=True)
        tq2.gate_up_swiglu(soa, soa, x[:1], n, k, out=o["swiglu1"])
        tq2.gate_up_swiglu(soa, soa, x, n, k, out=o["swiglu40"])
        tq2.gemv(soa_q1, xq[0], n, k, out=o["q1gemv"], fmt="q1")
        tq2.gemm(soa_q1, xq, n, k, out=o["q1gemm"], fmt="q1")

    calls()
    torch.cuda.synchronize()
    eager = {name: t.clone() for name, t in outs.items()}

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        calls()                                 # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            calls()
    torch.cuda.synchronize()

    other = torch.empty(8, n, device="cuda")
    for replay in range(3):
        for t in outs.values():
            t.fill_(float("nan"))
        tq2.gemm(soa, x[8:16] * (replay + 2.0), n, k, out=other)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t in outs.items():
            print("replay", replay, name, flush=True)
            assert torch.equal(t, eager[name]), "replay %d: %s differs from eager" % (replay, name)
