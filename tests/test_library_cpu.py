"""CPU checks of libtq2: it loads, exports every symbol of include/tq2.h, and
its host-side logic (sizes, path choice, argument checks) behaves as the
header says.  No kernel is launched: every call below either is a pure host
function or is rejected before any device work."""

import ctypes
import os
import re

import pytest

from gemv_tq2_g128_amd import tq2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    with open(os.path.join(ROOT, "include", "tq2.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq2_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert len(names) == 20
    assert sorted(tq2.EXPORTED_SYMBOLS) == names
    lib = ctypes.CDLL(tq2.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name


def test_sizes():
    assert tq2.aos_bytes(1, 128) == 34
    assert tq2.aos_bytes(2, 128) == 68 == tq2.aos_bytes(1, 256)
    assert tq2.aos_bytes(4096, 4096) == 4456448
    assert tq2.aos_bytes(11008, 4096) == 11976704
    assert tq2.aos_bytes(3072, 3072) == 2506752
    for bad in [(1, 100), (1, 0), (-1, 128), (1, -128)]:
        assert tq2.aos_bytes(*bad) == 0 and tq2.soa_bytes(*bad) == 0
    for n, k in [(1, 128), (3, 384), (4096, 4096), (11008, 4096), (77, 12288)]:
        s = tq2.soa_bytes(n, k)
        assert s % 256 == 0
        assert s >= n * k // 4 + n * (k // 128) * 2
        assert s < n * k // 4 + n * (k // 128) * 2 + 512
    assert tq2.soa_layout_version() == 1


def test_gemm_path():
    assert tq2.gemm_path(1, 4096, 4096) == tq2.PATH_GEMV
    for m in (2, 7, 8, 9, 16):
        assert tq2.gemm_path(m, 11008, 4096) == tq2.PATH_SPLIT_F16
    for m in (17, 100, 1536):
        assert tq2.gemm_path(m, 3072, 3072) == tq2.PATH_F16
    assert tq2.gemm_path(8, 10, 100) == tq2.TQ2_ERR_SHAPE
    assert tq2.gemm_path(8, 10, 0) == tq2.TQ2_ERR_INVALID
    assert tq2.gemm_path(-1, 10, 128) == tq2.TQ2_ERR_INVALID
    assert tq2.gemm_path(8, 10, 1 << 31) == tq2.TQ2_ERR_INVALID


def test_status_strings():
    for st in range(0, -7, -1):
        s = tq2.status_string(st)
        assert s and s != "unknown tq2 status"
    assert tq2.status_string(-99) == "unknown tq2 status"


# Fake, never-dereferenced addresses: every call below fails its host-side
# checks before the library touches the device.
A = 0x7F0000000000          # 256-byte aligned


def test_argument_checks_before_any_device_work():
    g, v, r = tq2.gemm_ptr, tq2.gemv_ptr, tq2.reformat_aos_to_soa_ptr
    assert g(A, A + 0x100000, 0, A + 0x200000, 4, 8, 100) == tq2.TQ2_ERR_SHAPE
    assert g(A, A + 0x100000, 0, A + 0x200000, 4, 8, 0) == tq2.TQ2_ERR_INVALID
    assert g(A, A + 0x100000, 0, A + 0x200000, -4, 8, 128) == tq2.TQ2_ERR_INVALID
    assert g(0, A + 0x100000, 0, A + 0x200000, 4, 8, 128) == tq2.TQ2_ERR_INVALID
    assert g(A, 0, 0, A + 0x200000, 4, 8, 128) == tq2.TQ2_ERR_INVALID
    assert g(A, A + 0x100000, 0, 0, 4, 8, 128) == tq2.TQ2_ERR_INVALID
    assert g(A + 64, A + 0x100000, 0, A + 0x200000, 4, 8, 128) == tq2.TQ2_ERR_ALIGN
    assert g(A, A + 0x100004, 0, A + 0x200000, 4, 8, 128) == tq2.TQ2_ERR_ALIGN
    assert g(A, A + 0x100000, A + 0x300008, A + 0x200000, 4, 8, 128) == tq2.TQ2_ERR_ALIGN
    # out overlapping x, the weight, or part of the residual
    assert g(A, A + 0x100000, 0, A + 0x100000 + 16, 4, 8, 128) == tq2.TQ2_ERR_ALIAS
    assert g(A, A + 0x100000, 0, A + 16 * 16, 4, 8, 128) == tq2.TQ2_ERR_ALIAS
    assert g(A, A + 0x100000, A + 0x200010, A + 0x200000, 4, 8, 128) == tq2.TQ2_ERR_ALIAS
    assert v(A, A + 0x100000, 0, A + 0x100000, 8, 128) == tq2.TQ2_ERR_ALIAS
    assert v(A, A + 0x100000, 0, A + 0x200000, 8, 200) == tq2.TQ2_ERR_SHAPE
    assert r(A + 1, A + 0x100000, 8, 128) == tq2.TQ2_ERR_ALIGN
    assert r(A, A + 0x100010, 8, 128) == tq2.TQ2_ERR_ALIGN
    assert r(A, A, 8, 128) == tq2.TQ2_ERR_ALIAS
    assert r(0, A, 8, 128) == tq2.TQ2_ERR_INVALID
    # empty shapes are no-ops that touch nothing, even with null pointers
    pg = tq2.gemm_precise_ptr
    assert pg(A, A + 0x100000, 0, A + 0x200000, 4, 8, 100) == tq2.TQ2_ERR_SHAPE
    assert pg(A + 64, A + 0x100000, 0, A + 0x200000, 4, 8, 128) == tq2.TQ2_ERR_ALIGN
    assert pg(A, A + 0x100000, 0, A + 0x100000, 4, 8, 128) == tq2.TQ2_ERR_ALIAS
    assert pg(0, 0, 0, 0, 0, 8, 128) == tq2.TQ2_OK
    assert g(0, 0, 0, 0, 0, 8, 128) == tq2.TQ2_OK
    assert g(0, 0, 0, 0, 4, 0, 128) == tq2.TQ2_OK
    assert v(0, 0, 0, 0, 0, 128) == tq2.TQ2_OK
    assert r(0, 0, 0, 128) == tq2.TQ2_OK


def test_gemm_workspace_sizes_and_checks():
    """tq2_gemm_workspace_bytes: nonzero exactly on path 2 up to M = 128, x as
    binary16 with rows padded to 16 and K to 256; tq2_gemm_ws rejects a
    missing, small, misaligned or overlapping workspace before any device
    work, and with no workspace needed it is tq2_gemm (same checks)."""
    wb = tq2.gemm_workspace_bytes
    for m in (1, 2, 16, 129, 1536):
        assert wb(m, 11008, 4096) == 0
    assert wb(17, 64, 128) == 2 * 16 * 256 * 2
    assert wb(100, 11008, 4096) == 7 * 16 * 4096 * 2
    assert wb(128, 50, 12416) == 8 * 16 * 12544 * 2
    assert wb(100, 10, 100) == 0 and wb(-1, 10, 128) == 0 and wb(0, 10, 128) == 0
    assert wb(40, 16, (1 << 21) + 128) == 0                    # K past the matrix-core limit
    w = tq2.gemm_ws_ptr
    X, O, W = A + (1 << 40), A + (2 << 40), A + (3 << 40)
    need = wb(100, 64, 4096)
    assert w(A, X, 0, O, 100, 64, 4096, 0, need) == tq2.TQ2_ERR_INVALID
    assert w(A, X, 0, O, 100, 64, 4096, W, need - 1) == tq2.TQ2_ERR_INVALID
    assert w(A, X, 0, O, 100, 64, 4096, W + 16, need) == tq2.TQ2_ERR_ALIGN
    assert w(A, X, 0, O, 100, 64, 4096, X + 256, need) == tq2.TQ2_ERR_ALIAS
    assert w(A, X, 0, O, 100, 64, 4096, O, need) == tq2.TQ2_ERR_ALIAS
    assert w(A, X, O + (1 << 30), O, 100, 64, 4096, O + (1 << 30), need) == tq2.TQ2_ERR_ALIAS
    assert w(A, X, 0, O, 100, 64, 4096, A, need) == tq2.TQ2_ERR_ALIAS
    assert w(A, X, 0, O, 100, 64, 100, W, need) == tq2.TQ2_ERR_SHAPE
    assert w(A + 64, X, 0, O, 100, 64, 4096, W, need) == tq2.TQ2_ERR_ALIGN
    assert w(A, X, 0, X + 16, 100, 64, 4096, W, need) == tq2.TQ2_ERR_ALIAS
    assert w(0, 0, 0, 0, 0, 64, 4096, 0, 0) == tq2.TQ2_OK
    # no workspace needed (M <= 16): the tq2_gemm checks, workspace ignored
    assert w(A, X, 0, X + 16, 8, 64, 4096, 0, 0) == tq2.TQ2_ERR_ALIAS


def test_noalloc_limits_before_any_device_work():
    """tq2_gemm_noalloc: the scratch size in the header is the binding's, a
    call that needs more workspace than it holds is INVALID before any
    device work, and the usual checks come first where they apply."""
    with open(os.path.join(ROOT, "include", "tq2.h")) as f:
        text = f.read()
    val = re.search(r"#define\s+TQ2_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", text)
    assert int(val.group(1)) << int(val.group(2)) == tq2.NOALLOC_SCRATCH_BYTES
    na = tq2.gemm_noalloc_ptr
    X, O = A + (1 << 40), A + (2 << 40)
    wb = tq2.gemm_workspace_bytes
    assert wb(100, 64, 18688) <= tq2.NOALLOC_SCRATCH_BYTES < wb(100, 64, 18944)
    assert wb(128, 64, 16384) <= tq2.NOALLOC_SCRATCH_BYTES < wb(128, 64, 16640)
    assert na(A, X, 0, O, 100, 64, 18944) == tq2.TQ2_ERR_INVALID
    assert na(A, X, 0, O, 128, 64, 16640) == tq2.TQ2_ERR_INVALID
    assert na(A, X, 0, O, 100, 64, 100) == tq2.TQ2_ERR_SHAPE
    assert na(A + 64, X, 0, O, 100, 64, 4096) == tq2.TQ2_ERR_ALIGN
    assert na(A, X, 0, X + 16, 100, 64, 4096) == tq2.TQ2_ERR_ALIAS
    assert na(A, X, 0, X + 16, 8, 64, 4096) == tq2.TQ2_ERR_ALIAS       # M <= 16: tq2_gemm
    assert na(0, 0, 0, 0, 0, 64, 4096) == tq2.TQ2_OK


def test_size_limits_before_any_device_work():
    """Dimensions above 2^30, and on the matrix-core paths K above 2^21 or
    N * K / 4 code bytes at 2^31 or more, are rejected before any device
    work (the buffers are far apart, so no alias check fires first)."""
    g, pg, v = tq2.gemm_ptr, tq2.gemm_precise_ptr, tq2.gemv_ptr
    X, O = A + (1 << 40), A + (2 << 40)
    big_k = (1 << 21) + 128
    assert g(A, X, 0, O, 2, 16, big_k) == tq2.TQ2_ERR_INVALID          # path 1
    assert g(A, X, 0, O, 40, 16, big_k) == tq2.TQ2_ERR_INVALID         # path 2
    assert pg(A, X, 0, O, 40, 16, big_k) == tq2.TQ2_ERR_INVALID
    assert g(A, X, 0, O, 2, 1 << 21, 4096) == tq2.TQ2_ERR_INVALID      # 2^31 code bytes
    assert g(A, X, 0, O, 40, 1 << 21, 4096) == tq2.TQ2_ERR_INVALID
    assert g(A, X, 0, O, (1 << 30) + 1, 8, 128) == tq2.TQ2_ERR_INVALID
    assert g(A, X, 0, O, 4, (1 << 30) + 1, 128) == tq2.TQ2_ERR_INVALID
    assert v(A, X, 0, O, (1 << 30) + 1, 128) == tq2.TQ2_ERR_INVALID
    assert v(A, X, 0, O, 8, (1 << 30) + 128) == tq2.TQ2_ERR_INVALID


def test_probe_library_for_the_benchmark():
    """libtq2_probe.so (reference launches for bench.py, built beside libtq2)
    exports its two entry points and rejects bad arguments before any launch."""
    import ctypes
    from gemv_tq2_g128_amd import build as B
    path = os.path.join(B.PKG_DIR, B.PROBE_LIB_NAME)
    assert os.path.exists(path), "run the build first"
    lib = ctypes.CDLL(path, mode=ctypes.RTLD_LOCAL)
    lib.tq2_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_int, ctypes.c_void_p]
    lib.tq2_probe_empty.argtypes = [ctypes.c_int, ctypes.c_void_p]
    assert lib.tq2_probe_read(None, 4096, A, 8, None) == -1
    assert lib.tq2_probe_read(A, 4096, None, 8, None) == -1
    assert lib.tq2_probe_read(A, 4100, A + 0x100000, 8, None) == -1
    assert lib.tq2_probe_read(A, 4096, A + 0x100000, 0, None) == -1
    assert lib.tq2_probe_empty(0, None) == -1


def test_batched_gemv_checks_before_any_device_work():
    b = tq2.gemv_batched_ptr
    X, O = A + 0x100000, A + 0x200000
    ok = (A, X, 0, O, 8, 128)
    assert b([]) == tq2.TQ2_OK
    assert tq2.lib.tq2_gemv_batched(None, 1, None) == tq2.TQ2_ERR_INVALID
    assert tq2.lib.tq2_gemv_batched(None, -1, None) == tq2.TQ2_ERR_INVALID
    assert b([ok] * (tq2.GEMV_BATCH_MAX + 1)) == tq2.TQ2_ERR_INVALID
    assert b([ok, (A, X, 0, O + 64, 8, 100)]) == tq2.TQ2_ERR_SHAPE
    assert b([ok, (A, X, 0, 0, 8, 128)]) == tq2.TQ2_ERR_INVALID
    assert b([ok, (A + 64, X, 0, O + 64, 8, 128)]) == tq2.TQ2_ERR_ALIGN
    assert b([(A, X, 0, X, 8, 128)]) == tq2.TQ2_ERR_ALIAS           # out over its own x
    # another problem's out over this problem's x, weight, out or residual
    assert b([ok, (A + 0x10000, X + 0x1000, 0, X, 8, 128)]) == tq2.TQ2_ERR_ALIAS
    assert b([ok, (A + 0x10000, X, 0, A + 16, 8, 128)]) == tq2.TQ2_ERR_ALIAS
    assert b([ok, (A + 0x10000, X, 0, O + 16, 8, 128)]) == tq2.TQ2_ERR_ALIAS
    assert b([(A, X, O + 0x100, O, 8, 128), (A, X, 0, O + 0x100, 8, 128)]) == tq2.TQ2_ERR_ALIAS
    # empty problems are skipped; an all-empty batch is a no-op
    assert b([(0, 0, 0, 0, 0, 128), (0, 0, 0, 0, 0, 256)]) == tq2.TQ2_OK
    # one k's problems whose grid (ceil(n / 4) row blocks each) would pass
    # 2^31 - 1 blocks: rejected before anything is enqueued, even after a
    # smaller k's group that fits (far-apart buffers, so no alias fires)
    big = [(A + (i << 38), A + (1 << 44) + (i << 38), 0, A + (2 << 44) + (i << 38), 1 << 30, 256)
           for i in range(8)]
    small = [(A + (3 << 44), A + (3 << 44) + (1 << 40), 0, A + (3 << 44) + (2 << 40), 8, 128)]
    assert b(small + big) == tq2.TQ2_ERR_INVALID


def test_swiglu_checks_before_any_device_work():
    sw = tq2.gate_up_swiglu_ptr
    U, X, O = A + 0x40000, A + 0x100000, A + 0x200000
    assert sw(A, U, X, O, 4, 8, 100) == tq2.TQ2_ERR_SHAPE
    assert sw(A, U, X, O, 4, 8, 0) == tq2.TQ2_ERR_INVALID
    assert sw(A, U, X, O, -1, 8, 128) == tq2.TQ2_ERR_INVALID
    for bad in [(0, U, X, O), (A, 0, X, O), (A, U, 0, O), (A, U, X, 0)]:
        assert sw(*bad, 4, 8, 128) == tq2.TQ2_ERR_INVALID
    assert sw(A + 64, U, X, O, 4, 8, 128) == tq2.TQ2_ERR_ALIGN
    assert sw(A, U + 64, X, O, 4, 8, 128) == tq2.TQ2_ERR_ALIGN
    assert sw(A, U, X + 4, O, 4, 8, 128) == tq2.TQ2_ERR_ALIGN
    assert sw(A, U, X, O + 4, 4, 8, 128) == tq2.TQ2_ERR_ALIGN
    # out over x, over the gate weight or over the up weight
    assert sw(A, U, X, X + 16, 4, 8, 128) == tq2.TQ2_ERR_ALIAS
    assert sw(A, U, X, A + 16, 4, 8, 128) == tq2.TQ2_ERR_ALIAS
    assert sw(A, U, X, U + 16, 4, 8, 128) == tq2.TQ2_ERR_ALIAS
    # K beyond the matrix-core kernels' limit (buffers spaced so nothing overlaps)
    assert sw(A, A + (1 << 24), A + (1 << 25), A + (1 << 27), 4, 8, 1 << 22) == \
        tq2.TQ2_ERR_INVALID
    assert sw(0, 0, 0, 0, 0, 8, 128) == tq2.TQ2_OK
    assert sw(0, 0, 0, 0, 4, 0, 128) == tq2.TQ2_OK


def test_q1_sizes_and_checks():
    assert tq2.q1_aos_bytes(1, 128) == 18
    assert tq2.q1_aos_bytes(4096, 4096) == 2359296
    for bad in [(1, 100), (1, 0), (-1, 128)]:
        assert tq2.q1_aos_bytes(*bad) == 0 and tq2.q1_soa_bytes(*bad) == 0
    for n, k in [(1, 128), (3, 384), (4096, 4096), (77, 12288)]:
        s = tq2.q1_soa_bytes(n, k)
        assert s % 256 == 0
        assert n * k // 8 + n * (k // 128) * 2 <= s < n * k // 8 + n * (k // 128) * 2 + 512
    r, v, g = tq2.q1_reformat_aos_to_soa_ptr, tq2.q1_gemv_ptr, tq2.q1_gemm_ptr
    X, O = A + 0x100000, A + 0x200000
    assert r(A + 1, X, 8, 128) == tq2.TQ2_ERR_ALIGN
    assert r(A + 0x1C0, A + 0x200, 8, 128) == tq2.TQ2_ERR_ALIAS     # 144 B of AoS over soa
    assert r(A, A + 160, 8, 128) == tq2.TQ2_ERR_ALIGN
    assert r(0, 0, 0, 128) == tq2.TQ2_OK
    assert v(A, X, 0, O, 8, 200) == tq2.TQ2_ERR_SHAPE
    assert v(A, X, 0, X, 8, 128) == tq2.TQ2_ERR_ALIAS
    assert g(A + 64, X, 0, O, 4, 8, 128) == tq2.TQ2_ERR_ALIGN
    # the Q1 weight (8 rows x 16 B of bits + scales, 512 B) vs out
    assert g(A, X, 0, A + 256, 4, 8, 128) == tq2.TQ2_ERR_ALIAS
    assert g(A, X, 0, A + 512, 4, 8, 128) != tq2.TQ2_ERR_ALIAS
    assert g(0, 0, 0, 0, 0, 8, 128) == tq2.TQ2_OK
    sw = tq2.q1_gate_up_swiglu_ptr
    assert sw(A, A + 0x40000, X, O, 4, 8, 100) == tq2.TQ2_ERR_SHAPE
    assert sw(A, A + 0x40000, X, A + 0x40000, 4, 8, 128) == tq2.TQ2_ERR_ALIAS


def test_device_check_without_gpu():
    """Valid arguments but no gfx950 device: the call must return
    TQ2_ERR_DEVICE (never crash).  Only meaningful where no GPU is visible."""
    torch = pytest.importorskip("torch")
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible; this check is for GPU-less hosts")
    st = tq2.gemm_ptr(A, A + 0x100000, 0, A + 0x200000, 4, 8, 128)
    assert st == tq2.TQ2_ERR_DEVICE
    assert tq2.q1_gemm_ptr(A, A + 0x100000, 0, A + 0x200000, 4, 8, 128) == tq2.TQ2_ERR_DEVICE
    assert tq2.q1_reformat_aos_to_soa_ptr(A, A + 0x100000, 8, 128) == tq2.TQ2_ERR_DEVICE
    # gate and up may be the same buffer
    assert tq2.gate_up_swiglu_ptr(A, A, A + 0x100000, A + 0x200000, 1, 8, 128) == \
        tq2.TQ2_ERR_DEVICE
    # shared x and weight, distinct outs: valid, so the device check decides
    st = tq2.gemv_batched_ptr([(A, A + 0x100000, 0, A + 0x200000, 8, 128),
                               (A, A + 0x100000, 0, A + 0x200100, 8, 128)])
    assert st == tq2.TQ2_ERR_DEVICE


def test_binding_requires_one_device():
    """The torch front end refuses tensors on different devices (a kernel only
    reaches memory of the device it runs on); None entries are skipped."""
    import torch
    a, b = torch.empty(1), torch.empty(1, device="meta")
    assert tq2._one_device(("x", a), ("residual", None), ("out", a)) == a.device
    with pytest.raises(ValueError, match="out is on meta"):
        tq2._one_device(("x", a), ("out", b))


def test_binding_mirrors_the_header():
    """The binding's status codes, batch limit and problem struct are the
    header's: values parsed from include/tq2.h, fields in declaration order
    with the same sizes (pointers and int64_t, no padding)."""
    with open(os.path.join(ROOT, "include", "tq2.h")) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    codes = dict((k, int(v)) for k, v in re.findall(r"\b(TQ2_(?:OK|ERR_[A-Z]+))\s*=\s*(-?\d+)", text))
    assert len(codes) == 7
    for name, value in codes.items():
        assert getattr(tq2, name) == value, name
    assert int(re.search(r"#define\s+TQ2_GEMV_BATCH_MAX\s+(\d+)", text).group(1)) == \
        tq2.GEMV_BATCH_MAX
    body = re.search(r"typedef struct tq2_gemv_problem \{(.*?)\}", text, flags=re.S).group(1)
    fields = re.findall(r"(\w+)\s*;", body)
    assert fields == [f[0] for f in tq2.GemvProblem._fields_]
    sizes = {"soa": 8, "x": 8, "residual": 8, "out": 8, "n": 8, "k": 8}
    for name, ctype in tq2.GemvProblem._fields_:
        assert ctypes.sizeof(ctype) == sizes[name], name
    assert ctypes.sizeof(tq2.GemvProblem) == 48
