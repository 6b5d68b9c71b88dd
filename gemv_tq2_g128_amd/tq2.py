"""Python binding of libtq2, the gfx950 TQ2_0_g128 ternary matmul.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libtq2.so``; PyTorch provides device memory and streams.  There
is no CPU fallback: importing this package fails loudly when the library has
not been built (``python -m gemv_tq2_g128_amd.build``).

The C entry points are declared in ``include/tq2.h``; the functions here have
the same names without the ``tq2_`` prefix.
"""

from __future__ import annotations

import ctypes
import os

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libtq2.so")

TQ2_OK = 0
TQ2_ERR_INVALID = -1
TQ2_ERR_SHAPE = -2
TQ2_ERR_ALIGN = -3
TQ2_ERR_ALIAS = -4
TQ2_ERR_DEVICE = -5
TQ2_ERR_LAUNCH = -6
NOALLOC_SCRATCH_BYTES = 4 << 20   # TQ2_NOALLOC_SCRATCH_BYTES (include/tq2.h)

GEMV_BATCH_MAX = 32

PATH_GEMV = 0
PATH_SPLIT_F16 = 1
PATH_F16 = 2

EXPORTED_SYMBOLS = (
    "tq2_aos_bytes",
    "tq2_soa_bytes",
    "tq2_soa_layout_version",
    "tq2_reformat_aos_to_soa",
    "tq2_gemv",
    "tq2_gemv_batched",
    "tq2_gemm",
    "tq2_gemm_workspace_bytes",
    "tq2_gemm_ws",
    "tq2_gemm_noalloc",
    "tq2_gemm_precise",
    "tq2_gate_up_swiglu",
    "tq2_q1_aos_bytes",
    "tq2_q1_soa_bytes",
    "tq2_q1_reformat_aos_to_soa",
    "tq2_q1_gemv",
    "tq2_q1_gemm",
    "tq2_q1_gate_up_swiglu",
    "tq2_gemm_path",
    "tq2_status_string",
)


class GemvProblem(ctypes.Structure):
    """Mirror of tq2_gemv_problem (include/tq2.h)."""
    _fields_ = [("soa", ctypes.c_void_p), ("x", ctypes.c_void_p), ("residual", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("n", ctypes.c_int64), ("k", ctypes.c_int64)]


def _hip_runtimes_mapped():
    """Distinct HIP runtime files mapped into this process (Linux)."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libtq2.so is not built (expected at %s); run "
            "`python -m gemv_tq2_g128_amd.build`" % LIB_PATH)
    # PyTorch ships its own HIP runtime.  Loading torch first makes libtq2's
    # dependency on libamdhip64.so.7 resolve to that same runtime (same
    # soname), so device pointers and streams from torch are valid in libtq2.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError("two HIP runtimes are loaded (%s); import torch before loading "
                          "libtq2 by any other route" % ", ".join(runtimes))
    i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    c_int = ctypes.c_int
    lib.tq2_aos_bytes.argtypes = [i64, i64]
    lib.tq2_aos_bytes.restype = sz
    lib.tq2_soa_bytes.argtypes = [i64, i64]
    lib.tq2_soa_bytes.restype = sz
    lib.tq2_soa_layout_version.argtypes = []
    lib.tq2_soa_layout_version.restype = c_int
    lib.tq2_reformat_aos_to_soa.argtypes = [vp, vp, i64, i64, vp]
    lib.tq2_reformat_aos_to_soa.restype = c_int
    lib.tq2_gemv.argtypes = [vp, vp, vp, vp, i64, i64, vp]
    lib.tq2_gemv.restype = c_int
    lib.tq2_gemv_batched.argtypes = [ctypes.POINTER(GemvProblem), c_int, vp]
    lib.tq2_gemv_batched.restype = c_int
    lib.tq2_gemm.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
    lib.tq2_gemm.restype = c_int
    lib.tq2_gemm_precise.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
    lib.tq2_gemm_precise.restype = c_int
    lib.tq2_gemm_workspace_bytes.argtypes = [i64, i64, i64]
    lib.tq2_gemm_workspace_bytes.restype = sz
    lib.tq2_gemm_ws.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, sz, vp]
    lib.tq2_gemm_ws.restype = c_int
    lib.tq2_gemm_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
    lib.tq2_gemm_noalloc.restype = c_int
    lib.tq2_gate_up_swiglu.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
    lib.tq2_gate_up_swiglu.restype = c_int
    lib.tq2_q1_aos_bytes.argtypes = [i64, i64]
    lib.tq2_q1_aos_bytes.restype = sz
    lib.tq2_q1_soa_bytes.argtypes = [i64, i64]
    lib.tq2_q1_soa_bytes.restype = sz
    lib.tq2_q1_reformat_aos_to_soa.argtypes = [vp, vp, i64, i64, vp]
    lib.tq2_q1_reformat_aos_to_soa.restype = c_int
    lib.tq2_q1_gemv.argtypes = [vp, vp, vp, vp, i64, i64, vp]
    lib.tq2_q1_gemv.restype = c_int
    lib.tq2_q1_gemm.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
    lib.tq2_q1_gemm.restype = c_int
    lib.tq2_q1_gate_up_swiglu.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
    lib.tq2_q1_gate_up_swiglu.restype = c_int
    lib.tq2_gemm_path.argtypes = [i64, i64, i64]
    lib.tq2_gemm_path.restype = c_int
    lib.tq2_status_string.argtypes = [c_int]
    lib.tq2_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()


class TQ2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


def _check(status: int, where: str) -> None:
    if status != TQ2_OK:
        raise TQ2Error(status, where)


# ---------------------------------------------------------------------------
# Host-only queries.
# ---------------------------------------------------------------------------

def aos_bytes(n: int, k: int) -> int:
    return int(lib.tq2_aos_bytes(n, k))


def soa_bytes(n: int, k: int) -> int:
    return int(lib.tq2_soa_bytes(n, k))


def q1_aos_bytes(n: int, k: int) -> int:
    return int(lib.tq2_q1_aos_bytes(n, k))


def q1_soa_bytes(n: int, k: int) -> int:
    return int(lib.tq2_q1_soa_bytes(n, k))


def _sizes(fmt: str):
    """(aos_bytes, soa_bytes) functions of a weight format ("tq2" or "q1")."""
    if fmt == "tq2":
        return aos_bytes, soa_bytes
    if fmt == "q1":
        return q1_aos_bytes, q1_soa_bytes
    raise ValueError("unknown weight format %r" % (fmt,))


def soa_layout_version() -> int:
    return int(lib.tq2_soa_layout_version())


def gemm_path(m: int, n: int, k: int) -> int:
    return int(lib.tq2_gemm_path(m, n, k))


def gemm_workspace_bytes(m: int, n: int, k: int) -> int:
    return int(lib.tq2_gemm_workspace_bytes(m, n, k))


def status_string(status: int) -> str:
    return lib.tq2_status_string(status).decode()


# ---------------------------------------------------------------------------
# Raw-pointer calls (device pointers and a hipStream_t as integers).
# ---------------------------------------------------------------------------

def reformat_aos_to_soa_ptr(aos_ptr: int, soa_ptr: int, n: int, k: int, stream: int = 0) -> int:
    return int(lib.tq2_reformat_aos_to_soa(aos_ptr, soa_ptr, n, k, stream or None))


def gemv_ptr(soa_ptr: int, x_ptr: int, residual_ptr: int, out_ptr: int, n: int, k: int,
             stream: int = 0) -> int:
    return int(lib.tq2_gemv(soa_ptr, x_ptr, residual_ptr or None, out_ptr, n, k, stream or None))


def gemv_batched_ptr(problems, stream: int = 0) -> int:
    """problems: sequence of (soa_ptr, x_ptr, residual_ptr or 0, out_ptr, n, k)."""
    arr = (GemvProblem * max(1, len(problems)))()
    for i, (soa_p, x_p, r_p, o_p, n, k) in enumerate(problems):
        arr[i] = GemvProblem(soa_p or None, x_p or None, r_p or None, o_p or None, n, k)
    return int(lib.tq2_gemv_batched(arr, len(problems), stream or None))


def gemm_ptr(soa_ptr: int, x_ptr: int, residual_ptr: int, out_ptr: int, m: int, n: int, k: int,
             stream: int = 0) -> int:
    return int(lib.tq2_gemm(soa_ptr, x_ptr, residual_ptr or None, out_ptr, m, n, k,
                            stream or None))


def gemm_ws_ptr(soa_ptr: int, x_ptr: int, residual_ptr: int, out_ptr: int, m: int, n: int, k: int,
                ws_ptr: int, ws_bytes: int, stream: int = 0) -> int:
    return int(lib.tq2_gemm_ws(soa_ptr, x_ptr, residual_ptr or None, out_ptr, m, n, k,
                               ws_ptr or None, ws_bytes, stream or None))


def gemm_noalloc_ptr(soa_ptr: int, x_ptr: int, residual_ptr: int, out_ptr: int, m: int, n: int,
                     k: int, stream: int = 0) -> int:
    return int(lib.tq2_gemm_noalloc(soa_ptr, x_ptr, residual_ptr or None, out_ptr, m, n, k,
                                    stream or None))


def gemm_precise_ptr(soa_ptr: int, x_ptr: int, residual_ptr: int, out_ptr: int, m: int, n: int,
                     k: int, stream: int = 0) -> int:
    return int(lib.tq2_gemm_precise(soa_ptr, x_ptr, residual_ptr or None, out_ptr, m, n, k,
                                    stream or None))


def q1_reformat_aos_to_soa_ptr(aos_ptr: int, soa_ptr: int, n: int, k: int,
                               stream: int = 0) -> int:
    return int(lib.tq2_q1_reformat_aos_to_soa(aos_ptr, soa_ptr, n, k, stream or None))


def q1_gemv_ptr(soa_ptr: int, x_ptr: int, residual_ptr: int, out_ptr: int, n: int, k: int,
                stream: int = 0) -> int:
    return int(lib.tq2_q1_gemv(soa_ptr, x_ptr, residual_ptr or None, out_ptr, n, k,
                               stream or None))


def q1_gemm_ptr(soa_ptr: int, x_ptr: int, residual_ptr: int, out_ptr: int, m: int, n: int,
                k: int, stream: int = 0) -> int:
    return int(lib.tq2_q1_gemm(soa_ptr, x_ptr, residual_ptr or None, out_ptr, m, n, k,
                               stream or None))


def q1_gate_up_swiglu_ptr(gate_ptr: int, up_ptr: int, x_ptr: int, out_ptr: int, m: int, n: int,
                          k: int, stream: int = 0) -> int:
    return int(lib.tq2_q1_gate_up_swiglu(gate_ptr or None, up_ptr or None, x_ptr or None,
                                         out_ptr or None, m, n, k, stream or None))


def gate_up_swiglu_ptr(gate_ptr: int, up_ptr: int, x_ptr: int, out_ptr: int, m: int, n: int,
                       k: int, stream: int = 0) -> int:
    return int(lib.tq2_gate_up_swiglu(gate_ptr or None, up_ptr or None, x_ptr or None,
                                      out_ptr or None, m, n, k, stream or None))


# ---------------------------------------------------------------------------
# torch.Tensor front end.
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_handle(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _require(t, dtype, numel: int, what: str):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % what)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % what)
    if t.dtype != dtype:
        raise ValueError("%s must have dtype %s, got %s" % (what, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % what)
    if t.numel() != numel:
        raise ValueError("%s must have %d elements, got %d" % (what, numel, t.numel()))


def _one_device(*named):
    """The device of the given (name, tensor) pairs, which must all be the
    same: a kernel reads and writes only memory of the device it runs on."""
    dev = None
    for what, t in named:
        if t is None:
            continue
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("%s is on %s, the other tensors on %s" % (what, t.device, dev))
    return dev


def _launch(dev, fn, *args):
    """Run a raw call with `dev` as the current device and its current stream:
    a launch on the null stream goes to the current device."""
    torch = _torch()
    with torch.cuda.device(dev):
        return fn(*args, _stream_handle(dev))


def reformat_aos_to_soa(aos, n: int, k: int, out=None, fmt: str = "tq2"):
    """AoS block bytes (uint8 device tensor) -> resident SoA weight (uint8).
    fmt: "tq2" (34-byte TQ2_0_g128 blocks) or "q1" (18-byte Q1_g128 blocks)."""
    torch = _torch()
    aos_b, soa_b = _sizes(fmt)
    nbytes = aos_b(n, k)
    if nbytes == 0 and n != 0:
        _check(TQ2_ERR_SHAPE if k > 0 else TQ2_ERR_INVALID, "reformat_aos_to_soa")
    _require(aos, torch.uint8, nbytes, "aos")
    if out is None:
        out = torch.empty(soa_b(n, k), dtype=torch.uint8, device=aos.device)
    _require(out, torch.uint8, soa_b(n, k), "soa")
    dev = _one_device(("aos", aos), ("soa", out))
    call = q1_reformat_aos_to_soa_ptr if fmt == "q1" else reformat_aos_to_soa_ptr
    _check(_launch(dev, call, aos.data_ptr(), out.data_ptr(), n, k), "reformat_aos_to_soa")
    return out


def gemv(soa, x, n: int, k: int, residual=None, out=None, fmt: str = "tq2"):
    """out[n] = residual[n] + sum_k x[k] * w[n, k]; x is f32 [k] (or [1, k])."""
    torch = _torch()
    _require(soa, torch.uint8, _sizes(fmt)[1](n, k), "soa")
    _require(x, torch.float32, k, "x")
    if residual is not None:
        _require(residual, torch.float32, n, "residual")
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=x.device)
    _require(out, torch.float32, n, "out")
    dev = _one_device(("x", x), ("soa", soa), ("residual", residual), ("out", out))
    call = q1_gemv_ptr if fmt == "q1" else gemv_ptr
    _check(_launch(dev, call, soa.data_ptr(), x.data_ptr(),
                   residual.data_ptr() if residual is not None else 0, out.data_ptr(), n, k),
           "gemv")
    return out


def gemm(soa, x, n: int, k: int, residual=None, out=None, precise: bool = False,
         fmt: str = "tq2", workspace="auto"):
    """out[m, n] = residual[m, n] + sum_k x[m, k] * w[n, k]; x is f32 [m, k].
    precise=True calls tq2_gemm_precise (f32-class accuracy at every M; TQ2
    only).  workspace (TQ2, not precise): "auto" calls tq2_gemm_ws with a
    workspace allocated here where tq2_gemm_workspace_bytes is nonzero; a
    uint8 device tensor is used as that workspace; None calls tq2_gemm."""
    torch = _torch()
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError("x must be [m, %d]" % k)
    if precise and fmt != "tq2":
        raise ValueError("precise=True is a TQ2 entry point")
    m = x.shape[0]
    _require(soa, torch.uint8, _sizes(fmt)[1](n, k), "soa")
    _require(x, torch.float32, m * k, "x")
    if residual is not None:
        _require(residual, torch.float32, m * n, "residual")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _require(out, torch.float32, m * n, "out")
    dev = _one_device(("x", x), ("soa", soa), ("residual", residual), ("out", out))
    res_ptr = residual.data_ptr() if residual is not None else 0
    if fmt == "tq2" and not precise and workspace is not None:
        need = gemm_workspace_bytes(m, n, k)
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError("workspace must be 'auto', None or a uint8 tensor")
            workspace = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        elif need:
            if not (isinstance(workspace, torch.Tensor) and workspace.dtype == torch.uint8
                    and workspace.is_contiguous() and workspace.device == dev):
                raise ValueError("workspace must be a contiguous uint8 tensor on %s" % dev)
        if need and workspace is not None:
            _check(_launch(dev, gemm_ws_ptr, soa.data_ptr(), x.data_ptr(), res_ptr,
                           out.data_ptr(), m, n, k, workspace.data_ptr(), workspace.numel()),
                   "gemm_ws")
            return out
    call = q1_gemm_ptr if fmt == "q1" else (gemm_precise_ptr if precise else gemm_ptr)
    _check(_launch(dev, call, soa.data_ptr(), x.data_ptr(), res_ptr, out.data_ptr(), m, n, k),
           "gemm_precise" if precise else "gemm")
    return out


def gemv_batched(problems):
    """Independent GEMVs in one call.  problems: sequence of dicts with keys
    soa, x, n, k and optional residual, out.  Returns the list of outs."""
    torch = _torch()
    if len(problems) == 0:
        return []
    raw, outs, dev = [], [], None
    for p in problems:
        n, k = p["n"], p["k"]
        _require(p["soa"], torch.uint8, soa_bytes(n, k), "soa")
        _require(p["x"], torch.float32, k, "x")
        res = p.get("residual")
        if res is not None:
            _require(res, torch.float32, n, "residual")
        out = p.get("out")
        if out is None:
            out = torch.empty(n, dtype=torch.float32, device=p["x"].device)
        _require(out, torch.float32, n, "out")
        d = _one_device(("x", p["x"]), ("soa", p["soa"]), ("residual", res), ("out", out))
        if dev is not None and d != dev:
            raise ValueError("every problem of one batch must be on one device")
        dev = d
        outs.append(out)
        raw.append((p["soa"].data_ptr(), p["x"].data_ptr(), res.data_ptr() if res is not None else 0,
                    out.data_ptr(), n, k))
    _check(_launch(dev, gemv_batched_ptr, raw), "gemv_batched")
    return outs


def gate_up_swiglu(gate_soa, up_soa, x, n: int, k: int, out=None, fmt: str = "tq2"):
    """out[m, n] = silu(x W_gate^T)[m, n] * (x W_up^T)[m, n]; x is f32 [m, k]."""
    torch = _torch()
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError("x must be [m, %d]" % k)
    m = x.shape[0]
    sb = _sizes(fmt)[1](n, k)
    _require(gate_soa, torch.uint8, sb, "gate_soa")
    _require(up_soa, torch.uint8, sb, "up_soa")
    _require(x, torch.float32, m * k, "x")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _require(out, torch.float32, m * n, "out")
    dev = _one_device(("x", x), ("gate_soa", gate_soa), ("up_soa", up_soa), ("out", out))
    call = q1_gate_up_swiglu_ptr if fmt == "q1" else gate_up_swiglu_ptr
    _check(_launch(dev, call, gate_soa.data_ptr(), up_soa.data_ptr(), x.data_ptr(),
                   out.data_ptr(), m, n, k), "gate_up_swiglu")
    return out
