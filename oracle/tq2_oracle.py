"""CPU oracle for the TQ2_0_g128 ternary matmul -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The GPU library never calls it and
shares no code, table or constant with it.

What it computes (oxibonsai-image 0.2.2, src/gpu.rs: module doc, "Correctness
contract", and the doc of ``ternary_matmul_gpu``)::

    out[m, n] = residual[m, n] + sum_k input[m, k] * dequant(W)[n, k]

for a row-major f32 ``input[M, K]``, out-major weight blocks ``[N, K]`` and a
row-major ``out[M, N]`` -- the plain ``A . B^T`` contraction with no transpose.
The residual term follows the ``*_residual`` kernels of the same kernel
library (oxibonsai-kernels 0.1.5, pipelines.rs: ``MetalPipelines`` fields
``gemv_q1_g128_v7_residual`` and ``gemm_q1_g128_v7_residual``), read as "add
the residual once to the finished dot product".

Block format (gpu.rs, doc of ``blocks_as_bytes``): 34 bytes, ``qs[32]`` then a
binary16 ``d``, little endian, no padding; ``N * (K / 128)`` blocks, row ``n``'s
blocks contiguous with the block index increasing with ``k``.

Readings where the pages are silent (recorded convention, shared with the
library only through this documentation):

* weight ``j`` (0..127) of a block has code ``(qs[j // 4] >> (2 * (j % 4))) & 3``
  (least significant bits first);
* codes map to values 0 -> -1, 1 -> 0, 2 -> +1; code 3 is reserved and
  decodes to 0;
* the weight is ``value(code) * d``.

Everything is evaluated in float64.  ``dequantize`` and the sums are written
out plainly; the large-size path uses NumPy's float64 matrix product as the
summation step, which the tests pin against the scalar triple loop.

Fused gate/up projections with SwiGLU (the ternary counterpart of the
``fused_gate_up_swiglu_q1`` / ``fused_gate_up_swiglu_gemm_q1`` pipelines of
oxibonsai-kernels 0.1.5, pipelines.rs, ``MetalPipelines``, decode and prefill
sections; their arithmetic is not printed, and the element-wise ``silu_f32``
pipeline of the same table names the activation)::

    out[m, n] = silu(g[m, n]) * u[m, n],   silu(z) = z / (1 + exp(-z)),
    g = x @ W_gate^T,  u = x @ W_up^T      (two [N, K] ternary weights)

read as the usual SwiGLU feed-forward gate: SiLU of the gate projection times
the up projection, element by element, with no residual.

Parity pins: the f16 decoder, block size, code map, bit order and the
contraction are pinned by ``tests/test_oracle.py``, and so are SiLU and the
gate/up composition.  The bit order and the
code map are the recorded convention above -- the pages print neither -- so
they are pinned to that convention, not to a worked example of the pages.
"""

from __future__ import annotations

import math

import numpy as np

BLOCK_WEIGHTS = 128          # weights per block ("g128")
BLOCK_BYTES = 34             # qs[32] + f16 d
CODE_BYTES = 32


# ---------------------------------------------------------------------------
# binary16 decoding, written from the IEEE 754 definition (1 sign bit, 5
# exponent bits with bias 15, 10 fraction bits; exponent 0 = zero/subnormal,
# exponent 31 = infinity/NaN).
# ---------------------------------------------------------------------------

def f16_bits_to_float(bits: int) -> float:
    """Decode one binary16 bit pattern to a Python float (exact)."""
    bits &= 0xFFFF
    sign = -1.0 if (bits >> 15) & 1 else 1.0
    exponent = (bits >> 10) & 0x1F
    fraction = bits & 0x3FF
    if exponent == 0:
        return sign * fraction * 2.0 ** -24          # zero or subnormal
    if exponent == 0x1F:
        return sign * math.inf if fraction == 0 else math.nan
    return sign * (1.0 + fraction / 1024.0) * 2.0 ** (exponent - 15)


def f16_bits_to_float_array(bits: np.ndarray) -> np.ndarray:
    """Element-wise ``f16_bits_to_float`` over a uint16 array, in float64."""
    b = bits.astype(np.int64) & 0xFFFF
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    exponent = (b >> 10) & 0x1F
    fraction = (b & 0x3FF).astype(np.float64)
    normal = (1.0 + fraction / 1024.0) * np.exp2((exponent - 15).astype(np.float64))
    sub = fraction * 2.0 ** -24
    special = np.where(fraction == 0, np.inf, np.nan)
    mag = np.where(exponent == 0, sub, np.where(exponent == 0x1F, special, normal))
    return sign * mag


# ---------------------------------------------------------------------------
# Ternary code map (recorded convention; see module docstring).
# ---------------------------------------------------------------------------

CODE_VALUE = {0: -1.0, 1: 0.0, 2: 1.0, 3: 0.0}


def code_of(qs: bytes, j: int) -> int:
    """2-bit code of weight ``j`` of a block's ``qs`` (least significant first)."""
    return (qs[j >> 2] >> (2 * (j & 3))) & 3


def aos_bytes(n: int, k: int) -> int:
    """Size of an ``[n, k]`` weight in AoS blocks."""
    return n * (k // BLOCK_WEIGHTS) * BLOCK_BYTES


# ---------------------------------------------------------------------------
# Scalar reference (pure Python; small inputs only).
# ---------------------------------------------------------------------------

def dequantize_block_scalar(block: bytes) -> list:
    """The 128 weights of one 34-byte block, as Python floats."""
    if len(block) != BLOCK_BYTES:
        raise ValueError("a block is 34 bytes")
    qs = block[:CODE_BYTES]
    d = f16_bits_to_float(block[32] | (block[33] << 8))
    return [CODE_VALUE[code_of(qs, j)] * d for j in range(BLOCK_WEIGHTS)]


def dequantize_scalar(aos: bytes, n: int, k: int) -> list:
    """``[n][k]`` weights from AoS bytes, block by block."""
    if k <= 0 or k % BLOCK_WEIGHTS:
        raise ValueError("k must be a positive multiple of 128")
    if len(aos) != aos_bytes(n, k):
        raise ValueError("weight byte length does not match n * (k/128) * 34")
    kb = k // BLOCK_WEIGHTS
    w = []
    for row in range(n):
        r = []
        for b in range(kb):
            off = (row * kb + b) * BLOCK_BYTES
            r.extend(dequantize_block_scalar(bytes(aos[off:off + BLOCK_BYTES])))
        w.append(r)
    return w


def matmul_scalar(aos: bytes, x, n: int, k: int, residual=None):
    """Triple loop: ``out[m][n] = residual[m][n] + sum_k x[m][k] * w[n][k]``,
    summed in increasing ``k`` in float64."""
    w = dequantize_scalar(aos, n, k)
    m_rows = len(x)
    out = []
    for m in range(m_rows):
        row = []
        for j in range(n):
            acc = 0.0
            for kk in range(k):
                acc += float(x[m][kk]) * w[j][kk]
            if residual is not None:
                acc = float(residual[m][j]) + acc
            row.append(acc)
        out.append(row)
    return out


# ---------------------------------------------------------------------------
# NumPy float64 reference (same definition, for realistic sizes).
# ---------------------------------------------------------------------------

def _blocks(aos: np.ndarray, n: int, k: int) -> np.ndarray:
    aos = np.asarray(aos, dtype=np.uint8).reshape(-1)
    if k <= 0 or k % BLOCK_WEIGHTS:
        raise ValueError("k must be a positive multiple of 128")
    if aos.size != aos_bytes(n, k):
        raise ValueError("weight byte length does not match n * (k/128) * 34")
    return aos.reshape(n, k // BLOCK_WEIGHTS, BLOCK_BYTES)


def dequantize(aos: np.ndarray, n: int, k: int, rows=None) -> np.ndarray:
    """float64 ``[n, k]`` (or ``[len(rows), k]``) dequantised weights.

    Same steps as ``dequantize_block_scalar``, applied to every block at once:
    for each weight position ``j`` take the byte ``j // 4``, shift by
    ``2 * (j % 4)``, mask two bits, map the code to its value and multiply by
    the block's decoded scale."""
    blk = _blocks(aos, n, k)
    if rows is not None:
        blk = blk[np.asarray(rows)]
    qs = blk[:, :, :CODE_BYTES]
    d_bits = blk[:, :, 32].astype(np.uint16) | (blk[:, :, 33].astype(np.uint16) << 8)
    d = f16_bits_to_float_array(d_bits)                               # [r, kb]
    value_of_code = np.array([CODE_VALUE[c] for c in range(4)])
    w = np.empty(qs.shape[:2] + (BLOCK_WEIGHTS,), dtype=np.float64)
    for j in range(BLOCK_WEIGHTS):
        codes = (qs[:, :, j >> 2] >> (2 * (j & 3))) & 3
        w[:, :, j] = value_of_code[codes] * d
    return w.reshape(w.shape[0], -1)


def _dequantizer(fmt: str):
    """Weight decoder for a format: "tq2" (TQ2_0_g128, this module) or "q1"
    (Q1_g128, ``q1_oracle``)."""
    if fmt == "tq2":
        return dequantize
    if fmt == "q1":
        from .q1_oracle import dequantize_q1
        return dequantize_q1
    raise ValueError("unknown weight format %r" % (fmt,))


def matmul(aos: np.ndarray, x: np.ndarray, n: int, k: int, residual=None,
           fmt: str = "tq2") -> np.ndarray:
    """float64 ``out = residual + x @ W^T`` (unrounded)."""
    x64 = np.asarray(x, dtype=np.float64).reshape(-1, k)
    w = _dequantizer(fmt)(aos, n, k)
    out = x64 @ w.T
    if residual is not None:
        out = np.asarray(residual, dtype=np.float64).reshape(out.shape) + out
    return out


def error_scale(aos: np.ndarray, x: np.ndarray, n: int, k: int, residual=None,
                fmt: str = "tq2") -> np.ndarray:
    """``S[m, n] = sum_k |x[m, k] * w[n, k]|`` (+ ``|residual[m, n]|`` when a
    residual is added: it is one more term of the same sum)."""
    x64 = np.abs(np.asarray(x, dtype=np.float64).reshape(-1, k))
    w = np.abs(_dequantizer(fmt)(aos, n, k))
    s = x64 @ w.T
    if residual is not None:
        s = s + np.abs(np.asarray(residual, dtype=np.float64).reshape(s.shape))
    return s


def matmul_entries(aos: np.ndarray, x: np.ndarray, n: int, k: int, rows, cols,
                   residual=None, fmt: str = "tq2"):
    """Reference and error scale for selected outputs ``(rows[i], cols[i])``,
    each computed on its own (for spot checks of full-size runs)."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    x64 = np.asarray(x, dtype=np.float64).reshape(-1, k)
    ucols, inv = np.unique(cols, return_inverse=True)
    w = _dequantizer(fmt)(aos, n, k, rows=ucols)                        # [u, k]
    wi = w[inv]                                                         # [s, k]
    xi = x64[rows]                                                      # [s, k]
    ref = np.sum(xi * wi, axis=1)
    s = np.sum(np.abs(xi * wi), axis=1)
    if residual is not None:
        r = np.asarray(residual, dtype=np.float64).reshape(x64.shape[0], n)[rows, cols]
        ref = r + ref
        s = s + np.abs(r)
    return ref, s


def matmul_rows(aos: np.ndarray, x: np.ndarray, n: int, k: int, cols, residual=None,
                fmt: str = "tq2"):
    """Reference and error scale for all rows of ``x`` at output columns ``cols``."""
    cols = np.asarray(cols)
    x64 = np.asarray(x, dtype=np.float64).reshape(-1, k)
    w = _dequantizer(fmt)(aos, n, k, rows=cols)
    ref = x64 @ w.T
    s = np.abs(x64) @ np.abs(w).T
    if residual is not None:
        r = np.asarray(residual, dtype=np.float64).reshape(x64.shape[0], n)[:, cols]
        ref = r + ref
        s = s + np.abs(r)
    return ref, s


# ---------------------------------------------------------------------------
# Fused gate/up projections + SwiGLU.
# ---------------------------------------------------------------------------

# Upper bound of |d silu / dz| over the reals: silu'(z) = s (1 + z (1 - s)) with
# s = 1 / (1 + exp(-z)) peaks at about 1.0998 near z = 2.4.
SILU_SLOPE_BOUND = 1.1


def silu(z):
    """SiLU ``z / (1 + exp(-z))`` in float64 (0 for z -> -inf, z for z -> +inf)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def gate_up_swiglu(aos_gate: np.ndarray, aos_up: np.ndarray, x: np.ndarray, n: int,
                   k: int, fmt: str = "tq2") -> np.ndarray:
    """float64 ``silu(x @ W_gate^T) * (x @ W_up^T)``, shape ``[M, n]``."""
    g = matmul(aos_gate, x, n, k, fmt=fmt)
    u = matmul(aos_up, x, n, k, fmt=fmt)
    return silu(g) * u


def _swiglu_scale(g, u, sg, su, tol):
    # |silu(g + dg) (u + du) - silu(g) u|
    #     <= |silu(g + dg) - silu(g)| |u + du| + |silu(g)| |du|
    #     <= tol * (SLOPE * sg * (|u| + tol * su) + |silu(g)| * su)
    # for |dg| <= tol * sg and |du| <= tol * su.
    return SILU_SLOPE_BOUND * sg * (np.abs(u) + tol * su) + np.abs(silu(g)) * su


def gate_up_swiglu_error_scale(aos_gate: np.ndarray, aos_up: np.ndarray, x: np.ndarray,
                               n: int, k: int, tol: float, fmt: str = "tq2") -> np.ndarray:
    """Scale ``E`` such that projections each within ``tol * sum_k |x w|`` of
    the exact values give an output within ``tol * E`` of the exact one."""
    g = matmul(aos_gate, x, n, k, fmt=fmt)
    u = matmul(aos_up, x, n, k, fmt=fmt)
    sg = error_scale(aos_gate, x, n, k, fmt=fmt)
    su = error_scale(aos_up, x, n, k, fmt=fmt)
    return _swiglu_scale(g, u, sg, su, tol)


def gate_up_swiglu_parts(aos_gate: np.ndarray, aos_up: np.ndarray, x: np.ndarray, n: int,
                         k: int, fmt: str = "tq2"):
    """``(g, u, Sg, Su)``: both projections and their ``sum_k |x w|`` scales,
    each weight decoded once (for large cases)."""
    x64 = np.asarray(x, dtype=np.float64).reshape(-1, k)
    parts = []
    for aos in (aos_gate, aos_up):
        w = _dequantizer(fmt)(aos, n, k)
        parts.append((x64 @ w.T, np.abs(x64) @ np.abs(w).T))
    (g, sg), (u, su) = parts
    return g, u, sg, su


def swiglu_from_parts(parts, tol: float):
    """Reference ``silu(g) * u`` and error scale ``E`` from ``gate_up_swiglu_parts``."""
    g, u, sg, su = parts
    return silu(g) * u, _swiglu_scale(g, u, sg, su, tol)


def gate_up_swiglu_entries(aos_gate: np.ndarray, aos_up: np.ndarray, x: np.ndarray, n: int,
                           k: int, rows, cols, tol: float, fmt: str = "tq2"):
    """Reference and error scale ``E`` for selected outputs ``(rows[i], cols[i])``."""
    g, sg = matmul_entries(aos_gate, x, n, k, rows, cols, fmt=fmt)
    u, su = matmul_entries(aos_up, x, n, k, rows, cols, fmt=fmt)
    return silu(g) * u, _swiglu_scale(g, u, sg, su, tol)
