"""Seeded random shape sweep through every entry point, against the oracle.

Shapes are drawn from a fixed seed so that every run checks the same cases:
M in [1, 300], N in [1, 700], K = 128 * [1, 40], residual on or off, both
weight formats, plus the fused gate/up + SwiGLU.  Each case is compared
element by element with the tolerance of the path the library reports
(tests/parity.py).
"""

import numpy as np
import pytest

import oracle
import tq2_inputs as G
from tests.parity import TOL, check, check_swiglu

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


def _shapes(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        m = int(rng.choice([1, 2, 5, 8, 15, 16, 17, 31, 33, 64, 65, 97, 128, 129, 200, 300]))
        n = int(rng.integers(1, 701))
        k = 128 * int(rng.integers(1, 41))
        if m * n * k <= 60_000_000:
            out.append((m, n, k, bool(rng.integers(0, 2))))
    return out


SHAPES = _shapes(20261202, 24)


@pytest.mark.parametrize("fmt", ["tq2", "q1"])
@pytest.mark.parametrize("m,n,k,res", SHAPES)
def test_random_matmul(tq2, fmt, m, n, k, res):
    seed = 100000 + m * 7 + n * 13 + k
    c = (G.random_case if fmt == "tq2" else G.random_case_q1)(seed, m, n, k, residual=res)
    print("sweep", fmt, c["name"], "residual" if res else "", flush=True)
    soa = tq2.reformat_aos_to_soa(_dev(c["aos"]), n, k, fmt=fmt)
    x = _dev(c["x"])
    r = _dev(c["residual"]) if res else None
    if m == 1:
        y = tq2.gemv(soa, x.reshape(-1), n, k, residual=None if r is None else r.reshape(-1),
                     fmt=fmt)
        path = 0
    else:
        y = tq2.gemm(soa, x, n, k, residual=r, fmt=fmt)
        path = tq2.gemm_path(m, n, k)
    torch.cuda.synchronize()
    ref = oracle.matmul(c["aos"], c["x"], n, k, c["residual"], fmt=fmt)
    s = oracle.error_scale(c["aos"], c["x"], n, k, c["residual"], fmt=fmt)
    ok, msg = check(y.cpu().numpy().reshape(m, n), ref, s, path, c["name"])
    assert ok, msg


@pytest.mark.parametrize("fmt", ["tq2", "q1"])
@pytest.mark.parametrize("m,n,k,res", SHAPES[:12])
def test_random_swiglu(tq2, fmt, m, n, k, res):
    seed = 200000 + m * 7 + n * 13 + k
    make = G.swiglu_case if fmt == "tq2" else G.swiglu_case_q1
    c = make(seed, m, n, k)
    print("sweep swiglu", fmt, c["name"], flush=True)
    gs = tq2.reformat_aos_to_soa(_dev(c["gate"]), n, k, fmt=fmt)
    us = tq2.reformat_aos_to_soa(_dev(c["up"]), n, k, fmt=fmt)
    y = tq2.gate_up_swiglu(gs, us, _dev(c["x"]), n, k, fmt=fmt)
    torch.cuda.synchronize()
    path = tq2.gemm_path(m, n, k)
    ref, e = oracle.swiglu_from_parts(
        oracle.gate_up_swiglu_parts(c["gate"], c["up"], c["x"], n, k, fmt=fmt), TOL[path])
    ok, msg = check_swiglu(y.cpu().numpy().reshape(m, n), ref, e, path, c["name"])
    assert ok, msg


def test_random_gemm_precise(tq2):
    for m, n, k, res in SHAPES[:10]:
        c = G.random_case(300000 + m + n + k, m, n, k, residual=res)
        soa = tq2.reformat_aos_to_soa(_dev(c["aos"]), n, k)
        y = tq2.gemm(soa, _dev(c["x"]), n, k, residual=_dev(c["residual"]) if res else None,
                     precise=True)
        torch.cuda.synchronize()
        ref = oracle.matmul(c["aos"], c["x"], n, k, c["residual"])
        s = oracle.error_scale(c["aos"], c["x"], n, k, c["residual"])
        ok, msg = check(y.cpu().numpy().reshape(m, n), ref, s, 1, c["name"] + "_precise")
        assert ok, msg
