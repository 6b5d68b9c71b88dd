"""GPU parity of the Q1_g128 (1-bit) entry points against the CPU oracle.

Same kernels and tolerances as the TQ2 paths (tests/parity.py): path 0 and
path 1 within 1e-5 * sum_k |x w| (+ |residual|), path 2 within 2e-3 * S with
row cosine >= 0.99999; the fused gate/up + SwiGLU within the bound of
``check_swiglu``.  Inputs come from ``tq2_inputs`` (fair random bits, binary16
scales), references from ``oracle`` with ``fmt="q1"``.
"""

import numpy as np
import pytest

import oracle
import tq2_inputs as G
from tests.parity import check, check_swiglu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {0: 1e-5, 1: 1e-5, 2: 2e-3}


@pytest.fixture(scope="module")
def tq2():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    from gemv_tq2_g128_amd import tq2 as mod
    return mod


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def upload(tq2, aos, n, k):
    return tq2.reformat_aos_to_soa(_dev(aos), n, k, fmt="q1")


def host_soa_q1(aos, n, k):
    """Q1 SoA built on the host from the layout description in
    tq2_internal.h: bits plane [n][k/8] of 32-bit words, the bit of
    k = 32w + t at bit (t >> 1) + 16 (t & 1); binary16 scales [n][k/128] at
    align256(n k / 8); total rounded up to 256."""
    blk = aos.reshape(n * (k // 128), 18)
    bits = np.unpackbits(blk[:, :16].reshape(-1), bitorder="little").reshape(-1, 32)
    t = np.arange(32)
    shift = ((t >> 1) + 16 * (t & 1)).astype(np.uint32)
    words = np.bitwise_or.reduce(bits.astype(np.uint32) << shift[None, :], axis=1).astype("<u4")
    code_bytes = words.view(np.uint8)
    off = (code_bytes.size + 255) // 256 * 256
    total = (off + n * (k // 128) * 2 + 255) // 256 * 256
    out = np.zeros(total, dtype=np.uint8)
    out[: code_bytes.size] = code_bytes
    out[off: off + n * (k // 128) * 2] = blk[:, 16:].reshape(-1)
    return out


@pytest.mark.parametrize("n,k,seed", [(1, 128, 1), (3, 384, 2), (17, 1024, 3), (64, 4096, 4)])
def test_q1_reformat_matches_layout(tq2, n, k, seed):
    c = G.random_case_q1(seed, 1, n, k)
    got = upload(tq2, c["aos"], n, k)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    want = host_soa_q1(c["aos"], n, k)
    assert got.size == want.size == tq2.q1_soa_bytes(n, k)
    off = (n * k // 8 + 255) // 256 * 256
    used = np.zeros(got.size, bool)
    used[: n * k // 8] = True
    used[off: off + n * (k // 128) * 2] = True
    assert np.array_equal(got[used], want[used])


def run(tq2, case, inplace=False):
    m, n, k = case["m"], case["n"], case["k"]
    soa = upload(tq2, case["aos"], n, k)
    x = _dev(case["x"].reshape(m, k))
    res = _dev(case["residual"].reshape(m, n)) if case["residual"] is not None else None
    if m == 1 and case.get("gemv"):
        out = res.clone().reshape(-1) if inplace else None
        y = tq2.gemv(soa, x.reshape(-1), n, k, residual=out if inplace else
                     (None if res is None else res.reshape(-1)), out=out, fmt="q1")
    else:
        out = res.clone() if inplace else None
        y = tq2.gemm(soa, x, n, k, residual=out if inplace else res, out=out, fmt="q1")
    torch.cuda.synchronize()
    return y.cpu().numpy().reshape(m, n)


def assert_q1(tq2, case, inplace=False):
    print("q1 case", case["name"], "inplace" if inplace else "", flush=True)
    got = run(tq2, case, inplace)
    n, k = case["n"], case["k"]
    ref = oracle.matmul(case["aos"], case["x"], n, k, case["residual"], fmt="q1")
    s = oracle.error_scale(case["aos"], case["x"], n, k, case["residual"], fmt="q1")
    path = 0 if case["m"] == 1 else tq2.gemm_path(case["m"], n, k)
    ok, msg = check(got, ref, s, path, case["name"])
    print(msg, flush=True)
    assert ok, msg


Q1_GEMV_SHAPES = [(1, 128), (5, 256), (63, 384), (64, 1024), (65, 2176), (300, 4096),
                  (129, 8192), (77, 12288), (33, 16384), (40, 20480)]


@pytest.mark.parametrize("n,k", Q1_GEMV_SHAPES)
def test_q1_gemv_shapes(tq2, n, k):
    c = dict(G.random_case_q1(7000 + n + k, 1, n, k, residual=True), gemv=True)
    assert_q1(tq2, c)


def test_q1_decode_workload(tq2):
    for res in (False, True):
        c = dict(G.q1_decode(res), gemv=True)
        assert_q1(tq2, c)
    assert_q1(tq2, dict(G.q1_decode(True), gemv=True), inplace=True)


# Path 1 (M <= 16) scales x by a power of two per wave and K pass before the
# hi/lo split (the same skinny kernel as TQ2), so 1e-5 holds at any magnitude.
@pytest.mark.parametrize("m", [3, 8, 13])
@pytest.mark.parametrize("scale", [1e-6, 3e4])
def test_q1_split_path_x_magnitudes(tq2, m, scale):
    c = G.random_case_q1(9500 + m, m, 200, 1280, residual=True)
    c["x"] = (c["x"] * np.float32(scale)).astype(np.float32)
    c["residual"] = (c["residual"] * np.float32(scale)).astype(np.float32)
    c["name"] = "q1_x_scale_%g_m%d" % (scale, m)
    assert_q1(tq2, c)


def test_q1_split_path_passes_with_different_scales(tq2):
    """K = 8320: x 1e-3 in the first 4096-wide pass and 10 after it."""
    c = G.random_case_q1(9600, 8, 150, 8320, residual=True)
    x = c["x"].copy()
    x[:, :4096] *= np.float32(1e-3)
    x[:, 4096:] *= np.float32(10.0)
    c["x"] = x
    c["name"] = "q1_pass_scales_m8"
    assert_q1(tq2, c)


Q1_GEMM_SHAPES = [(2, 17, 128), (9, 100, 384), (16, 257, 1024), (5, 4100, 4224), (12, 8200, 2176),
                  (17, 200, 384), (33, 100, 256),
                  (64, 129, 384), (100, 300, 1024), (128, 64, 256), (129, 191, 384),
                  (200, 385, 768), (300, 1000, 1152), (150, 50, 12416), (64, 50, 12416)]


@pytest.mark.parametrize("m,n,k", Q1_GEMM_SHAPES)
def test_q1_gemm_shapes(tq2, m, n, k):
    c = G.random_case_q1(8000 + m + n + k, m, n, k, residual=True)
    assert_q1(tq2, c)
    assert_q1(tq2, dict(c, residual=None, name=c["name"] + "_nores"))


def test_q1_gemm_workload(tq2):
    assert_q1(tq2, G.q1_gemm())


@pytest.mark.parametrize("m", [1, 4, 40, 200])
def test_q1_special_bits_and_scales(tq2, m):
    base = G.random_case_q1(8500 + m, m, 96, 512, residual=True)
    a = base["aos"].reshape(-1, 18)
    for label, qs, d_bits in [("all_set", 0xFF, None), ("all_clear", 0x00, None),
                              ("neg_scale", None, 0xB800), ("zero_scale", None, 0x0000),
                              ("neg_zero_scale", None, 0x8000), ("subnormal", None, 0x0001),
                              ("d_max", None, 0x7BFF)]:
        b = a.copy()
        if qs is not None:
            b[:, :16] = qs
        if d_bits is not None:
            b[:, 16] = d_bits & 0xFF
            b[:, 17] = d_bits >> 8
        c = dict(base, aos=b.reshape(-1), name="q1_%s_m%d" % (label, m), gemv=(m == 1))
        assert_q1(tq2, c)


SWIGLU_Q1 = [(1, 300, 4096), (1, 77, 12288), (1, 63, 384), (1, 5, 256), (9, 100, 384),
             (5, 4100, 4224), (40, 130, 640), (200, 97, 768), (129, 191, 1024),
             (150, 50, 12416)]


@pytest.mark.parametrize("m,n,k", SWIGLU_Q1)
def test_q1_swiglu(tq2, m, n, k):
    c = G.swiglu_case_q1(9000 + m + n + k, m, n, k)
    print("q1 swiglu", c["name"], flush=True)
    gs, us = upload(tq2, c["gate"], n, k), upload(tq2, c["up"], n, k)
    y = tq2.gate_up_swiglu(gs, us, _dev(c["x"]), n, k, fmt="q1")
    torch.cuda.synchronize()
    path = tq2.gemm_path(m, n, k)
    ref, e = oracle.swiglu_from_parts(
        oracle.gate_up_swiglu_parts(c["gate"], c["up"], c["x"], n, k, fmt="q1"), TOL[path])
    ok, msg = check_swiglu(y.cpu().numpy(), ref, e, path, c["name"])
    print(msg, flush=True)
    assert ok, msg
