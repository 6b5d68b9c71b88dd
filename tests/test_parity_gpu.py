"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Every case draws seeded inputs from ``tq2_inputs``, runs the library on the
GPU and compares element by element with ``oracle`` (float64) within the
tolerance of the kernel path that ran (see tests/parity.py).
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


def upload_weight(tq2, aos, n, k):
    return tq2.reformat_aos_to_soa(_dev(aos), n, k)


def run_case(tq2, case, force_gemv=False, inplace=False, precise=False, workspace="auto"):
    m, n, k = case["m"], case["n"], case["k"]
    soa = upload_weight(tq2, case["aos"], n, k)
    x = _dev(case["x"].reshape(m, k))
    res = _dev(case["residual"].reshape(m, n)) if case["residual"] is not None else None
    out = res.clone() if (inplace and res is not None) else None
    res_arg = out if inplace and res is not None else res
    if force_gemv:
        assert m == 1
        y = tq2.gemv(soa, x.reshape(-1), n, k, residual=None if res_arg is None else res_arg.reshape(-1),
                     out=None if out is None else out.reshape(-1))
    else:
        y = tq2.gemm(soa, x, n, k, residual=res_arg, out=out, precise=precise,
                     workspace=workspace)
    torch.cuda.synchronize()
    return y.cpu().numpy().reshape(m, n)


def oracle_full(case):
    ref = oracle.matmul(case["aos"], case["x"], case["n"], case["k"], case["residual"])
    s = oracle.error_scale(case["aos"], case["x"], case["n"], case["k"], case["residual"])
    return ref, s


def assert_case(tq2, case, **kw):
    print("case", case["name"], kw, flush=True)
    got = run_case(tq2, case, **kw)
    ref, s = oracle_full(case)
    if kw.get("force_gemv") or case["m"] == 1:
        path = 0
    elif kw.get("precise"):
        path = 1
    else:
        path = tq2.gemm_path(case["m"], case["n"], case["k"])
    ok, msg = check(got, ref, s, path, case["name"])
    print(msg, flush=True)
    assert ok, msg
    return got


# ---------------------------------------------------------------------------
# Reformat: byte-exact against the documented private layout (version 1).
# ---------------------------------------------------------------------------

def host_soa_v1(aos, n, k):
    """SoA v1 built on the host from the layout description in tq2_internal.h:
    codes plane [n][k/4] with the code of k = 16w + t of word w at bit
    2*(t>>1) + 16*(t&1), code 3 stored as 1; binary16 scales [n][k/128] at
    align256(n*k/4); total rounded up to 256."""
    blk = aos.reshape(n * (k // 128), 34)
    qs = blk[:, :32].reshape(-1)
    bits = np.unpackbits(qs, bitorder="little").reshape(-1, 16, 2)   # [words, t, bit]
    codes = bits[:, :, 0].astype(np.uint32) | (bits[:, :, 1].astype(np.uint32) << 1)
    codes = np.where(codes == 3, 1, codes)
    t = np.arange(16)
    shift = (2 * (t >> 1) + 16 * (t & 1)).astype(np.uint32)
    words = np.bitwise_or.reduce(codes << shift[None, :], axis=1).astype("<u4")
    code_bytes = words.view(np.uint8)
    off = (code_bytes.size + 255) // 256 * 256
    total = (off + n * (k // 128) * 2 + 255) // 256 * 256
    out = np.zeros(total, dtype=np.uint8)
    out[: code_bytes.size] = code_bytes
    out[off: off + n * (k // 128) * 2] = blk[:, 32:].reshape(-1)
    return out


@pytest.mark.parametrize("n,k,seed", [(1, 128, 1), (3, 384, 2), (17, 1024, 3), (64, 4096, 4)])
def test_reformat_matches_layout(tq2, n, k, seed):
    assert tq2.soa_layout_version() == 1
    case = G.random_case(seed, 1, n, k, probs=(0.3, 0.3, 0.3, 0.1))   # includes code 3
    soa = upload_weight(tq2, case["aos"], n, k)
    torch.cuda.synchronize()
    got = soa.cpu().numpy()
    want = host_soa_v1(case["aos"], n, k)
    assert got.size == want.size == tq2.soa_bytes(n, k)
    off = (n * k // 4 + 255) // 256 * 256
    used = np.zeros(got.size, bool)
    used[: n * k // 4] = True
    used[off: off + n * (k // 128) * 2] = True
    assert np.array_equal(got[used], want[used])


# ---------------------------------------------------------------------------
# The five workloads at their full sizes.
# ---------------------------------------------------------------------------

def test_config1_gemv(tq2):
    c = G.config1()
    assert_case(tq2, c, force_gemv=True)
    assert_case(tq2, c)


def test_config2_gemv(tq2):
    assert_case(tq2, G.config2(False), force_gemv=True)


def test_config2_gemv_residual(tq2):
    c = G.config2(True)
    assert_case(tq2, c, force_gemv=True)
    assert_case(tq2, c, force_gemv=True, inplace=True)


@pytest.mark.parametrize("m", [7, 8, 9, 100])
def test_config3_gemm(tq2, m):
    assert_case(tq2, G.config3(m))
    if m > 16:
        assert_case(tq2, G.config3(m), workspace=None)


def test_config4_gemm(tq2):
    assert_case(tq2, G.config4())


def test_config5_chain_sampled(tq2):
    """100 chained layers at M=1536; every layer checked (teacher forced: the
    oracle consumes the GPU's actual layer input) on 48 sampled columns."""
    x = _dev(G.chain_input())
    rng = np.random.default_rng(55)
    for layer in range(G.CHAIN_LAYERS):
        k, n = G.chain_layer_shape(layer)
        aos = G.chain_layer_weight(layer)
        soa = upload_weight(tq2, aos, n, k)
        y = tq2.gemm(soa, x, n, k)
        torch.cuda.synchronize()
        cols = rng.choice(n, size=48, replace=False)
        ref, s = oracle.matmul_rows(aos, x.cpu().numpy(), n, k, cols)
        got = y[:, torch.from_numpy(cols).cuda()].cpu().numpy()
        ok, msg = check(got, ref, s, tq2.gemm_path(G.CHAIN_M, n, k), "layer %d" % layer)
        assert ok, msg
        # next input: first 3072 columns, RMS-rescaled per row (harness glue)
        nxt = y[:, : G.chain_layer_shape(layer + 1)[0]]
        x = (nxt / torch.sqrt(torch.mean(nxt * nxt, dim=1, keepdim=True) + 1e-6)).contiguous()
        del soa


# ---------------------------------------------------------------------------
# Shapes: several tiles plus ragged tails in M, N and K.
# ---------------------------------------------------------------------------

GEMV_SHAPES = [(1, 128), (5, 256), (63, 384), (64, 1024), (65, 2176), (300, 4096),
               (129, 8192), (77, 12288), (33, 16384), (40, 20480)]


@pytest.mark.parametrize("n,k", GEMV_SHAPES)
def test_gemv_shapes(tq2, n, k):
    c = G.random_case(1000 + n + k, 1, n, k, residual=True)
    assert_case(tq2, c, force_gemv=True)


GEMM_SHAPES = [(2, 17, 128), (3, 100, 384), (8, 64, 256), (15, 65, 640), (16, 257, 1024),
               (17, 200, 384), (31, 33, 128), (32, 300, 512), (33, 100, 256), (64, 129, 384),
               (65, 64, 1024), (96, 192, 256), (97, 250, 640), (128, 300, 512),
               (129, 191, 384), (200, 385, 768), (300, 1000, 1152), (150, 50, 12416),
               (257, 200, 16512), (100, 90, 12416), (33, 70, 16640)]


@pytest.mark.parametrize("m,n,k", GEMM_SHAPES)
def test_gemm_shapes(tq2, m, n, k):
    c = G.random_case(2000 + m + n + k, m, n, k, residual=True)
    assert_case(tq2, c)
    c2 = dict(c, residual=None, name=c["name"] + "_nores")
    assert_case(tq2, c2)


# The skinny kernel (M <= 16): every tiles-per-block instantiation (N up to
# 16 400, so the grid also exceeds 256 blocks), a ragged last block, one to
# four passes over K with partial last slices and chunks, both sides of the
# M = 8 packing limit, and the in-place residual.
SKINNY_SHAPES = [(8, 1, 128), (2, 300, 12416), (5, 4100, 4224), (9, 33, 4096),
                 (12, 8200, 2176), (16, 12290, 8320), (7, 16400, 1024), (16, 4096, 4096)]


@pytest.mark.parametrize("m,n,k", SKINNY_SHAPES)
def test_skinny_shapes(tq2, m, n, k):
    assert tq2.gemm_path(m, n, k) == 1
    c = G.random_case(2500 + m + n + k, m, n, k, residual=True)
    assert_case(tq2, c)


def test_skinny_inplace_residual(tq2):
    c = G.random_case(2601, 6, 4100, 4224, residual=True)
    assert_case(tq2, c, inplace=True)


# ---------------------------------------------------------------------------
# Edge values and degenerate cases.
# ---------------------------------------------------------------------------

def _blocks_with(case, qs_byte=None, d_bits=None):
    a = case["aos"].reshape(-1, 34).copy()
    if qs_byte is not None:
        a[:, :32] = qs_byte
    if d_bits is not None:
        a[:, 32] = d_bits & 0xFF
        a[:, 33] = d_bits >> 8
    return dict(case, aos=a.reshape(-1))


@pytest.mark.parametrize("m", [1, 4, 40])
def test_special_codes_and_scales(tq2, m):
    base = G.random_case(77 + m, m, 48, 512, residual=True)
    for label, kw in [("code3", dict(qs_byte=0xFF)), ("all_zero_weight", dict(qs_byte=0x55)),
                      ("all_plus", dict(qs_byte=0xAA)), ("all_minus", dict(qs_byte=0x00)),
                      ("d_zero", dict(d_bits=0x0000)), ("d_negative", dict(d_bits=0xB400)),
                      ("d_subnormal", dict(d_bits=0x0003)), ("d_max", dict(d_bits=0x7BFF))]:
        c = dict(_blocks_with(base, **kw), name="%s_m%d" % (label, m))
        assert_case(tq2, c)


def test_zero_weight_gives_residual_exactly(tq2):
    c = _blocks_with(G.random_case(5, 3, 40, 256, residual=True), qs_byte=0x55)
    got = run_case(tq2, c)
    assert np.array_equal(got, c["residual"].reshape(3, 40))
    c1 = _blocks_with(G.random_case(6, 1, 40, 256, residual=True), qs_byte=0x55)
    assert np.array_equal(run_case(tq2, c1, force_gemv=True), c1["residual"].reshape(1, 40))


def test_large_activations_f16_range(tq2):
    c = G.random_case(9, 64, 96, 256)
    c["x"] = (c["x"] * np.float32(8000.0)).astype(np.float32)     # |x| up to ~4e4 < 65504
    assert_case(tq2, c)


# The split-binary16 paths (M <= 16, and tq2_gemm_precise at any M) scale x
# by a power of two before the split (per wave and K pass in the skinny
# kernel, per x row in the tile kernel), so the 1e-5 tolerance holds at any
# magnitude of x: without it the lo limb of |x| below about 3e-3 falls into
# binary16's subnormal range.
@pytest.mark.parametrize("m", [1, 5, 8, 13, 40])
@pytest.mark.parametrize("scale", [1e-6, 2e-8, 3e4])
def test_split_paths_x_magnitudes(tq2, m, scale):
    c = G.random_case(8800 + m, m, 300, 1280, residual=True)
    c["x"] = (c["x"] * np.float32(scale)).astype(np.float32)
    c["residual"] = (c["residual"] * np.float32(scale)).astype(np.float32)
    c["name"] = "x_scale_%g_m%d" % (scale, m)
    if m <= 16:
        assert_case(tq2, c)                      # path 1 (or the GEMV at M = 1)
    assert_case(tq2, c, precise=True)


@pytest.mark.parametrize("m", [6, 12, 64])
def test_split_paths_rows_of_different_magnitude(tq2, m):
    """Row i of x scaled by 10^-(i % 5): four decades between rows."""
    c = G.random_case(8900 + m, m, 200, 640, residual=False)
    f = (10.0 ** -(np.arange(m) % 5)).astype(np.float32)[:, None]
    c["x"] = (c["x"] * f).astype(np.float32)
    c["name"] = "rows_magnitudes_m%d" % m
    if m <= 16:
        assert_case(tq2, c)
    assert_case(tq2, c, precise=True)


def test_split_tile_exponent_across_chunks(tq2):
    """tq2_gemm_precise at M = 64, K = 1536 (six 256-wide chunks): half the
    rows start with two all-zero chunks and are 1e-5 after them; the other
    rows grow tenfold per chunk, so the running exponent of a row falls from
    chunk to chunk and its sums are rescaled each time."""
    c = G.random_case(9100, 64, 130, 1536, residual=True)
    x = c["x"].copy()
    x[0::2, :512] = 0.0
    x[0::2, 512:] *= np.float32(1e-5)
    grow = (10.0 ** np.repeat(np.arange(6) - 3, 256)).astype(np.float32)
    x[1::2] *= grow[None, :]
    c["x"] = x
    c["name"] = "tile_exponent_across_chunks"
    assert_case(tq2, c, precise=True)


@pytest.mark.parametrize("m", [3, 8, 11, 16])
def test_skinny_passes_with_different_scales(tq2, m):
    """K = 8320: two full 4096-wide passes and a partial one, x 1e-3 in the
    first pass and 10 in the rest, so each pass takes its own power of two and
    the accumulators are rescaled between passes."""
    c = G.random_case(9000 + m, m, 150, 8320, residual=True)
    x = c["x"].copy()
    x[:, :4096] *= np.float32(1e-3)
    x[:, 4096:] *= np.float32(10.0)
    c["x"] = x
    c["name"] = "skinny_pass_scales_m%d" % m
    assert_case(tq2, c)


@pytest.mark.parametrize("m", [3, 8, 12, 40])
def test_split_paths_falling_then_rising_magnitude(tq2, m):
    """K = 12416: x about 1e16 in the first 4096-wide pass, 1e-16 in the
    second and 1 in the rest.  The split kernels' power of two only falls (it
    follows the largest |x| seen so far), so the large first pass is not
    scaled up past the f32 range when the tiny second pass arrives; the
    result is within 1e-5 * S, S dominated by the first pass.  M <= 16 runs
    the skinny kernel (tq2_gemm and tq2_gemm_precise), M = 40 the precise
    tile kernel (the binary16 path cannot hold 1e16)."""
    c = G.random_case(9050 + m, m, 140, 12416, residual=True)
    x = c["x"].copy()
    x[:, :4096] *= np.float32(1e16)
    x[:, 4096:8192] *= np.float32(1e-16)
    c["x"] = x
    c["residual"] = (c["residual"] * np.float32(1e16)).astype(np.float32)
    c["name"] = "split_falling_rising_m%d" % m
    if m <= 16:
        assert_case(tq2, c)
    assert_case(tq2, c, precise=True)


def test_gemm_m1536_k16384_sampled(tq2):
    """M = 1536, K = 16384 -> N = 3072 (an FFN down-projection shape, K above
    the 12288 of the 100-layer chain) on the M > 128 kernel: every row of 64
    sampled output columns, plus the in-place residual on the same columns."""
    m, n, k = 1536, 3072, 16384
    rng = np.random.default_rng(9600)
    aos = G.make_weight(rng, n, k)
    x = G.make_activations(rng, m, k, outlier_frac=0.01)
    res = rng.standard_normal((m, n), dtype=np.float32)
    soa = upload_weight(tq2, aos, n, k)
    cols = np.sort(rng.choice(n, size=64, replace=False))
    idx = torch.from_numpy(cols).cuda()
    xd = _dev(x)
    for with_res in (False, True):
        print("m1536 k16384 residual=%s" % with_res, flush=True)
        out = _dev(res) if with_res else None
        y = tq2.gemm(soa, xd, n, k, residual=out, out=out)
        torch.cuda.synchronize()
        got = y[:, idx].cpu().numpy()
        ref, s = oracle.matmul_rows(aos, x, n, k, cols, residual=res if with_res else None)
        ok, msg = check(got, ref, s, tq2.gemm_path(m, n, k), "m1536_k16384 res=%s" % with_res)
        print(msg, flush=True)
        assert ok, msg


@pytest.mark.parametrize("m", [1, 2, 17])
def test_largest_k(tq2, m):
    """K = 2^21, the largest K the matrix-core kernels take (their 32-bit
    buffer offsets span up to 128 x rows of K f32): the GEMV, the skinny
    kernel (512 passes over K) and the tile kernels, plus the precise one."""
    c = G.random_case(9400 + m, m, 20, 1 << 21, residual=True)
    assert_case(tq2, c)
    if m > 1:
        assert_case(tq2, c, precise=True)


@pytest.mark.parametrize("fmt", ["tq2", "q1"])
def test_largest_weight(tq2, fmt):
    """N = 2^21 - 1 rows at K = 4096: N * K / 4 = 2^31 - 1024, just under the
    limit the matrix-core kernels take (their buffer offsets are 32-bit; a
    TQ2 weight then has 2^31 - 1024 code bytes).  The rows repeat with a
    prime period of 4099, so an offset that wrapped or lost its high bits
    would read another row.  Sampled rows (the first, the last, both sides of
    period boundaries and the middle) are checked against the oracle on every
    path: GEMV, skinny, 16-column tile, ping-pong and precise, and for TQ2 the
    fused SwiGLU (gate = up) at M = 1 and M = 40."""
    n, k, period = (1 << 21) - 1, 4096, 4099
    q1 = fmt == "q1"
    row_bytes = (k // 128) * (18 if q1 else 34)
    make = G.make_weight_q1 if q1 else G.make_weight
    base = make(np.random.default_rng(9500), period, k)
    aos = np.tile(base, -(-n // period))[: n * row_bytes]
    print("largest weight %s: n=%d k=%d, %d AoS bytes" % (fmt, n, k, aos.size), flush=True)
    soa = tq2.reformat_aos_to_soa(_dev(aos), n, k, fmt=fmt)
    del aos
    torch.cuda.synchronize()
    rows = np.array([0, 1, period - 1, period, n // 2, n // 2 + 1, n - period - 1, n - period]
                    + list(range(n - 64, n)))
    aos_rows = np.concatenate([base[(r % period) * row_bytes:(r % period + 1) * row_bytes]
                               for r in rows])
    idx = torch.from_numpy(rows).cuda()
    rng = np.random.default_rng(9501)
    cases = ((1, False), (2, False), (40, False), (200, False)) + (() if q1 else ((40, True),))
    for m, precise in cases:
        x = rng.standard_normal((m, k), dtype=np.float32)
        print("largest weight %s: m=%d precise=%s" % (fmt, m, precise), flush=True)
        if m == 1:
            y = tq2.gemv(soa, _dev(x).reshape(-1), n, k, fmt=fmt).reshape(1, n)
            path = 0
        else:
            y = tq2.gemm(soa, _dev(x), n, k, precise=precise, fmt=fmt)
            path = 1 if precise else tq2.gemm_path(m, n, k)
        torch.cuda.synchronize()
        got = y[:, idx].cpu().numpy()
        del y
        ref = oracle.matmul(aos_rows, x, len(rows), k, None, fmt=fmt)
        sc = oracle.error_scale(aos_rows, x, len(rows), k, None, fmt=fmt)
        ok, msg = check(got, ref, sc, path, "largest %s m=%d%s" % (fmt, m, " precise" * precise))
        print(msg, flush=True)
        assert ok, msg
    if q1:
        return
    for m in (1, 40):
        x = rng.standard_normal((m, k), dtype=np.float32)
        print("largest weight swiglu: m=%d" % m, flush=True)
        y = tq2.gate_up_swiglu(soa, soa, _dev(x), n, k)
        torch.cuda.synchronize()
        got = y[:, idx].cpu().numpy()
        del y
        path = tq2.gemm_path(m, n, k)
        ref, e = oracle.swiglu_from_parts(
            oracle.gate_up_swiglu_parts(aos_rows, aos_rows, x, len(rows), k), TOL[path])
        ok, msg = check_swiglu(got, ref, e, path, "largest swiglu m=%d" % m)
        print(msg, flush=True)
        assert ok, msg


def test_empty_shapes_are_noops(tq2):
    soa = upload_weight(tq2, G.random_case(1, 1, 8, 128)["aos"], 8, 128)
    x = torch.zeros((0, 128), device="cuda")
    y = tq2.gemm(soa, x, 8, 128)
    assert y.shape == (0, 8)
    out = torch.full((4,), 7.0, device="cuda")
    assert tq2.gemm_ptr(soa.data_ptr(), x.data_ptr(), 0, out.data_ptr(), 4, 0, 128) == 0
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_deterministic_and_stream_aware(tq2):
    c = G.random_case(31, 37, 211, 640, residual=True)
    a = run_case(tq2, c)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = run_case(tq2, c)
    assert np.array_equal(a, b)


def test_error_codes_with_device_pointers(tq2):
    n, k, m = 32, 256, 4
    soa = upload_weight(tq2, G.random_case(2, 1, n, k)["aos"], n, k)
    x = torch.randn(m * k + 4, device="cuda")
    out = torch.empty(m * n + 4, device="cuda")
    res = torch.randn(m * n + 4, device="cuda")
    p = tq2.gemm_ptr
    assert p(soa.data_ptr(), x.data_ptr() + 4, 0, out.data_ptr(), m, n, k) == tq2.TQ2_ERR_ALIGN
    assert p(soa.data_ptr() + 16, x.data_ptr(), 0, out.data_ptr(), m, n, k) == tq2.TQ2_ERR_ALIGN
    assert p(soa.data_ptr(), x.data_ptr(), 0, x.data_ptr(), m, n, k) == tq2.TQ2_ERR_ALIAS
    assert p(soa.data_ptr(), x.data_ptr(), res.data_ptr() + 16, res.data_ptr(), m, n, k) == \
        tq2.TQ2_ERR_ALIAS
    assert p(soa.data_ptr(), x.data_ptr(), 0, out.data_ptr(), m, n, 100) == tq2.TQ2_ERR_SHAPE
    assert p(soa.data_ptr(), x.data_ptr(), 0, out.data_ptr(), -1, n, k) == tq2.TQ2_ERR_INVALID
    assert p(0, x.data_ptr(), 0, out.data_ptr(), m, n, k) == tq2.TQ2_ERR_INVALID
    assert p(soa.data_ptr(), x.data_ptr(), res.data_ptr(), res.data_ptr(), m, n, k) == tq2.TQ2_OK
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# Batched decode GEMV: independent problems in one call (one launch per k).
# ---------------------------------------------------------------------------

def _batched_check(tq2, specs, label):
    """specs: list of (n, k, with_residual, x_from, inplace); x_from = index of
    an earlier problem whose x this one shares, or None."""
    cases, probs = [], []
    for i, (n, k, with_res, x_from, inplace) in enumerate(specs):
        c = G.random_case(5000 + 7 * i + n + k, 1, n, k, residual=with_res)
        if x_from is not None:
            c = dict(c, x=cases[x_from]["x"])
        soa = upload_weight(tq2, c["aos"], n, k)
        x = probs[x_from]["x"] if x_from is not None else _dev(c["x"].reshape(-1))
        p = dict(soa=soa, x=x, n=n, k=k)
        if with_res:
            res = _dev(c["residual"].reshape(-1))
            p["residual"] = res
            if inplace:
                p["out"] = res
        cases.append(c)
        probs.append(p)
    print("batched case", label, [(c["n"], c["k"]) for c in cases], flush=True)
    outs = tq2.gemv_batched(probs)
    torch.cuda.synchronize()
    for c, y in zip(cases, outs):
        ref, s = oracle_full(c)
        ok, msg = check(y.cpu().numpy().reshape(1, -1), ref, s, 0, "%s_n%d_k%d" % (label, c["n"], c["k"]))
        print(msg, flush=True)
        assert ok, msg


def test_gemv_batched_mixed(tq2):
    specs = [(300, 1024, False, None, False), (4096, 1024, True, None, False),
             (77, 1024, False, 0, False), (1000, 4096, True, None, True), (9, 128, True, None, True),
             (513, 4096, False, 3, False), (40, 20480, True, None, False)]
    _batched_check(tq2, specs, "mixed")


def test_gemv_batched_full_batch(tq2):
    specs = [(64 + 5 * i, 128 * (1 + i % 3), i % 2 == 0, None, False)
             for i in range(tq2.GEMV_BATCH_MAX)]
    _batched_check(tq2, specs, "full")


def test_gemv_batched_matches_oracle_at_decode_size(tq2):
    specs = [(4096, 4096, True, None, False), (4096, 4096, True, 0, False),
             (4096, 4096, False, 0, False)]
    _batched_check(tq2, specs, "decode")


def test_gemv_batched_ragged(tq2):
    """Rows off the block size, K = 1152 (72 words per row: two 128-lane row
    slots per block, masked lanes), with and without residual, some in place."""
    specs = [(3700 + 13 * i, 1152, i % 3 != 2, None, i % 3 == 0) for i in range(9)]
    _batched_check(tq2, specs, "ragged")


# ---------------------------------------------------------------------------
# tq2_gemm_precise: f32-class accuracy (1e-5 * S) at every M.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("m,n,k", [(1, 300, 1024), (2, 77, 384), (17, 200, 384), (64, 129, 1024),
                                   (65, 300, 640), (100, 1000, 4096), (129, 191, 384)])
def test_gemm_precise_shapes(tq2, m, n, k):
    c = G.random_case(3000 + m + n + k, m, n, k, residual=True)
    assert_case(tq2, c, precise=True)


def test_gemm_precise_config3_m100(tq2):
    assert_case(tq2, dict(G.config3(100), name="config3_m100_precise"), precise=True)


def test_gemm_precise_config4(tq2):
    assert_case(tq2, dict(G.config4(), name="config4_precise"), precise=True)


# ---------------------------------------------------------------------------
# tq2_gate_up_swiglu: silu(x W_gate^T) * (x W_up^T), both projections fused.
# ---------------------------------------------------------------------------



def run_swiglu(tq2, case):
    m, n, k = case["m"], case["n"], case["k"]
    gs = upload_weight(tq2, case["gate"], n, k)
    us = gs if case.get("same") else upload_weight(tq2, case["up"], n, k)
    x = _dev(case["x"].reshape(m, k))
    y = tq2.gate_up_swiglu(gs, us, x, n, k)
    torch.cuda.synchronize()
    return y.cpu().numpy().reshape(m, n)


def swiglu_path(tq2, m, n, k):
    return tq2.gemm_path(m, n, k)


def assert_swiglu(tq2, case):
    print("swiglu case", case["name"], flush=True)
    m, n, k = case["m"], case["n"], case["k"]
    up = case["gate"] if case.get("same") else case["up"]
    got = run_swiglu(tq2, case)
    path = swiglu_path(tq2, m, n, k)
    ref = oracle.gate_up_swiglu(case["gate"], up, case["x"], n, k)
    e = oracle.gate_up_swiglu_error_scale(case["gate"], up, case["x"], n, k,
                                          {0: 1e-5, 1: 1e-5, 2: 2e-3}[path])
    ok, msg = check_swiglu(got, ref, e, path, case["name"])
    print(msg, flush=True)
    assert ok, msg
    return got, ref


SWIGLU_GEMV_SHAPES = [(1, 128), (5, 256), (63, 384), (64, 1024), (300, 4096), (77, 12288),
                      (40, 20480)]


@pytest.mark.parametrize("n,k", SWIGLU_GEMV_SHAPES)
def test_swiglu_decode_shapes(tq2, n, k):
    assert_swiglu(tq2, G.swiglu_case(4000 + n + k, 1, n, k))


# M = 2..16: split-binary16 kernel; 17..128: the warp-specialised kernel;
# > 128: the ping-pong kernel (K > 12288: scales loaded per chunk in both).
SWIGLU_GEMM_SHAPES = [(2, 17, 128), (9, 100, 384), (16, 257, 1024), (5, 4100, 4224),
                      (12, 8200, 2176), (17, 33, 256),
                      (40, 130, 640), (64, 96, 384), (100, 191, 1024), (129, 191, 384),
                      (200, 97, 768), (300, 1000, 1152), (150, 50, 12416), (100, 70, 12416)]


@pytest.mark.parametrize("m,n,k", SWIGLU_GEMM_SHAPES)
def test_swiglu_gemm_shapes(tq2, m, n, k):
    assert_swiglu(tq2, G.swiglu_case(5000 + m + n + k, m, n, k))


# Path 2 at 16 < M <= 128 runs one row block of the smallest 32-row multiple
# covering M (32 ... 128 rows): every tile height, at and just past its edge,
# and both sides of M = 104, up to which the 128-row tile stages 104 rows.
@pytest.mark.parametrize("m", [17, 31, 32, 33, 40, 48, 49, 63, 64, 65, 81, 96, 97, 100, 104,
                               105, 113, 127, 128])
def test_tile_heights(tq2, m):
    c = G.random_case(9200 + m, m, 150, 640, residual=(m % 2 == 0))
    assert_case(tq2, c)


# tq2_gemm_ws (16 < M <= 128): tq2.gemm uses it by default; the same shapes
# through tq2_gemm itself (no workspace) keep the warp-specialised kernel
# covered.  K <= 12288 stages the block's weights in LDS (K = 12288 fills
# it); K = 12416 and 16640 take the per-chunk weight loads.
WS_SHAPES = [(17, 200, 384), (31, 33, 128), (32, 300, 512), (33, 100, 256), (64, 129, 384),
             (65, 64, 1024), (96, 192, 256), (97, 250, 640), (100, 90, 12416), (104, 70, 4096),
             (105, 49, 1152), (128, 300, 512), (33, 70, 16640), (77, 100, 12288)]


@pytest.mark.parametrize("m,n,k", WS_SHAPES)
def test_path2_with_and_without_workspace(tq2, m, n, k):
    c = G.random_case(2500 + m + n + k, m, n, k, residual=(m % 2 == 1))
    assert tq2.gemm_workspace_bytes(m, n, k) > 0
    a = assert_case(tq2, c)                          # tq2_gemm_ws
    b = assert_case(tq2, c, workspace=None)          # tq2_gemm
    assert a.shape == b.shape


def test_workspace_contents_do_not_matter(tq2):
    """The pre-pass writes every workspace byte the GEMM reads (rows past M
    and k past K as zeros): a workspace full of binary16 NaNs beforehand, and
    one reused by a second, smaller call, give the oracle's results."""
    m, n, k = 100, 130, 1152
    need = tq2.gemm_workspace_bytes(m, n, k)
    ws = torch.full((need + 4096,), 0xFF, dtype=torch.uint8, device="cuda")
    for mm, kk in ((m, k), (37, 640)):
        c = G.random_case(2600 + mm, mm, n, kk, residual=True)
        soa = upload_weight(tq2, c["aos"], n, kk)
        x = _dev(c["x"].reshape(mm, kk))
        res = _dev(c["residual"].reshape(mm, n))
        y = tq2.gemm(soa, x, n, kk, residual=res, workspace=ws)
        torch.cuda.synchronize()
        ref, sc = oracle_full(c)
        ok, msg = check(y.cpu().numpy(), ref, sc, 2, c["name"] + "_ws")
        print(msg, flush=True)
        assert ok, msg
        assert np.isfinite(y.cpu().numpy()).all()


def test_workspace_in_place_residual_and_repeat(tq2):
    """In-place residual through tq2_gemm_ws, and two calls on the same
    inputs give identical bits (fixed reduction order)."""
    c = G.random_case(2700, 100, 96, 4096, residual=True)
    assert_case(tq2, c, inplace=True)
    soa = upload_weight(tq2, c["aos"], 96, 4096)
    x = _dev(c["x"].reshape(100, 4096))
    y1 = tq2.gemm(soa, x, 96, 4096)
    y2 = tq2.gemm(soa, x, 96, 4096)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("m", [17, 33, 49, 81, 105, 128])
def test_swiglu_tile_heights(tq2, m):
    assert_swiglu(tq2, G.swiglu_case(9300 + m, m, 70, 384))


def test_swiglu_same_weight_and_zero_gate(tq2):
    c = G.swiglu_case(6001, 40, 72, 512)
    got, _ = assert_swiglu(tq2, dict(c, same=True, name="same_weight"))
    assert np.all(got >= 0)                          # silu(u) * u >= 0
    zg = c["gate"].reshape(-1, 34).copy()
    zg[:, :32] = 0x55                                # every gate weight 0 -> g = 0 exactly
    for m in (1, 5, 40, 200):
        cz = G.swiglu_case(6002 + m, m, 72, 512)
        got = run_swiglu(tq2, dict(cz, gate=zg.reshape(-1), name="zero_gate_m%d" % m))
        assert np.all(got == 0), m


def test_swiglu_saturated_gate(tq2):
    # Large scales: |g| reaches the hundreds, so exp(-g) overflows or
    # vanishes in f32 and silu(g) must come out as 0 or g.
    for m in (1, 8, 64, 200):
        c = G.swiglu_case(6100 + m, m, 130, 1024, probs=G.UNIFORM_TERNARY, d_range=(2.0, 4.0))
        assert_swiglu(tq2, dict(c, name="saturated_m%d" % m))


def test_swiglu_feed_forward_workload(tq2):
    """K = 4096 -> N = 11008 at M = 1 (GEMV), 7 (split-binary16) and 100
    (binary16 matrix cores); the reference rows are the first M rows of one
    oracle evaluation over 100 activation rows (rows are independent)."""
    gate, up = G.swiglu_weights()
    n, k = G.SWIGLU_N, G.SWIGLU_K
    x = G.swiglu_activations(100)
    parts = oracle.gate_up_swiglu_parts(gate, up, x, n, k)
    gs, us = upload_weight(tq2, gate, n, k), upload_weight(tq2, up, n, k)
    for m in (1, 7, 100):
        print("swiglu workload m", m, flush=True)
        y = tq2.gate_up_swiglu(gs, us, _dev(x[:m]), n, k)
        torch.cuda.synchronize()
        path = tq2.gemm_path(m, n, k)
        ref, e = oracle.swiglu_from_parts(parts, {0: 1e-5, 1: 1e-5, 2: 2e-3}[path])
        ok, msg = check_swiglu(y.cpu().numpy(), ref[:m], e[:m], path, "workload m%d" % m)
        print(msg, flush=True)
        assert ok, msg


def test_swiglu_feed_forward_m1536_sampled(tq2):
    """K = 4096 -> N = 11008 at M = 1536 (the ping-pong kernel at full size):
    every column of 64 sampled rows, and 4096 scattered outputs."""
    gate, up = G.swiglu_weights()
    n, k, m = G.SWIGLU_N, G.SWIGLU_K, 1536
    x = G.swiglu_activations(m)
    gs, us = upload_weight(tq2, gate, n, k), upload_weight(tq2, up, n, k)
    got = tq2.gate_up_swiglu(gs, us, _dev(x), n, k)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    rng = np.random.default_rng(77)
    rows = np.sort(rng.choice(m, size=64, replace=False))
    ref, e = oracle.swiglu_from_parts(oracle.gate_up_swiglu_parts(gate, up, x[rows], n, k), 2e-3)
    ok, msg = check_swiglu(got[rows], ref, e, 2, "m1536 rows")
    print(msg, flush=True)
    assert ok, msg
    ri, ci = rng.integers(0, m, 4096), rng.integers(0, n, 4096)
    ref, e = oracle.gate_up_swiglu_entries(gate, up, x, n, k, ri, ci, 2e-3)
    ok, msg = check_swiglu(got[ri, ci], ref, e, 2, "m1536 scattered")
    print(msg, flush=True)
    assert ok, msg


def test_swiglu_error_codes_with_device_pointers(tq2):
    c = G.swiglu_case(6200, 4, 64, 256)
    gs = upload_weight(tq2, c["gate"], 64, 256)
    us = upload_weight(tq2, c["up"], 64, 256)
    x = _dev(c["x"])
    out = torch.empty((4, 64), dtype=torch.float32, device="cuda")
    sw = tq2.gate_up_swiglu_ptr
    assert sw(gs.data_ptr(), us.data_ptr(), x.data_ptr(), out.data_ptr(), 4, 64, 200) == \
        tq2.TQ2_ERR_SHAPE
    assert sw(gs.data_ptr(), us.data_ptr(), x.data_ptr(), x.data_ptr(), 4, 64, 256) == \
        tq2.TQ2_ERR_ALIAS
    assert sw(gs.data_ptr(), us.data_ptr() + 16, x.data_ptr(), out.data_ptr(), 4, 64, 256) == \
        tq2.TQ2_ERR_ALIGN
    assert sw(gs.data_ptr(), us.data_ptr(), x.data_ptr(), out.data_ptr(), 4, 64, 256) == tq2.TQ2_OK
    torch.cuda.synchronize()
