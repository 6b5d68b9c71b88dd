"""CPU oracle for the Q1_g128 (1-bit, group-128) sibling format -- TEST
INFRASTRUCTURE ONLY (same import rule as ``tq2_oracle``).

The pages name the 1-bit kernels -- ``gemv_q1_g128_v7`` (decode),
``gemv_q1_g128_v7_residual``, ``gemm_q1_g128_v7`` (prefill),
``gemm_q1_g128_v7_residual`` and the fused ``fused_gate_up_swiglu_q1`` /
``fused_gate_up_swiglu_gemm_q1`` (oxibonsai-kernels 0.1.5, pipelines.rs,
``MetalPipelines``, decode and prefill sections) -- but print neither the block
layout nor the bit-to-value map.  Readings taken here (recorded convention,
mirroring the TQ2_0_g128 block of oxibonsai-image 0.2.2, src/gpu.rs, doc of
``blocks_as_bytes``):

* a block holds 128 weights in 18 bytes: ``qs[16]`` (one bit per weight), then
  a little-endian binary16 scale ``d``; no padding; an ``[N, K]`` weight is
  ``N * (K / 128)`` blocks, row ``n``'s blocks contiguous in increasing ``k``;
* weight ``j`` (0..127) of a block has bit ``(qs[j // 8] >> (j % 8)) & 1``
  (least significant bit first);
* a set bit is ``+d`` and a clear bit is ``-d`` (weight ``(2 b - 1) d``).

The contraction, the residual and the fused gate/up + SwiGLU are the same
definitions as for TQ2 (see ``tq2_oracle``); ``tq2_oracle``'s matmul
functions take ``fmt="q1"`` to use this decoder.  Everything is float64.

Parity pins (``tests/test_oracle.py``): hand-worked blocks, the all-set and
all-clear closed forms, unit vectors over every bit position, the scalar
triple loop, and planted mistakes.  The layout and the sign map are pinned to
the recorded convention above, not to a printed example.
"""

from __future__ import annotations

import numpy as np

from .tq2_oracle import f16_bits_to_float, f16_bits_to_float_array

Q1_BLOCK_WEIGHTS = 128
Q1_BLOCK_BYTES = 18          # qs[16] + f16 d
Q1_CODE_BYTES = 16


def bit_of(qs: bytes, j: int) -> int:
    """Bit of weight ``j`` of a block's ``qs`` (least significant first)."""
    return (qs[j >> 3] >> (j & 7)) & 1


def q1_aos_bytes(n: int, k: int) -> int:
    """Size of an ``[n, k]`` Q1_g128 weight in AoS blocks."""
    return n * (k // Q1_BLOCK_WEIGHTS) * Q1_BLOCK_BYTES


def dequantize_block_scalar_q1(block: bytes) -> list:
    """The 128 weights of one 18-byte block, as Python floats."""
    if len(block) != Q1_BLOCK_BYTES:
        raise ValueError("a Q1_g128 block is 18 bytes")
    qs = block[:Q1_CODE_BYTES]
    d = f16_bits_to_float(block[16] | (block[17] << 8))
    return [(d if bit_of(qs, j) else -d) for j in range(Q1_BLOCK_WEIGHTS)]


def dequantize_scalar_q1(aos: bytes, n: int, k: int) -> list:
    """``[n][k]`` weights from Q1 AoS bytes, block by block."""
    if k <= 0 or k % Q1_BLOCK_WEIGHTS:
        raise ValueError("k must be a positive multiple of 128")
    if len(aos) != q1_aos_bytes(n, k):
        raise ValueError("weight byte length does not match n * (k/128) * 18")
    kb = k // Q1_BLOCK_WEIGHTS
    w = []
    for row in range(n):
        r = []
        for b in range(kb):
            off = (row * kb + b) * Q1_BLOCK_BYTES
            r.extend(dequantize_block_scalar_q1(bytes(aos[off:off + Q1_BLOCK_BYTES])))
        w.append(r)
    return w


def matmul_scalar_q1(aos: bytes, x, n: int, k: int, residual=None):
    """Triple loop over the Q1 weights, summed in increasing ``k`` in float64."""
    w = dequantize_scalar_q1(aos, n, k)
    out = []
    for m in range(len(x)):
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


def _blocks_q1(aos: np.ndarray, n: int, k: int) -> np.ndarray:
    aos = np.asarray(aos, dtype=np.uint8).reshape(-1)
    if k <= 0 or k % Q1_BLOCK_WEIGHTS:
        raise ValueError("k must be a positive multiple of 128")
    if aos.size != q1_aos_bytes(n, k):
        raise ValueError("weight byte length does not match n * (k/128) * 18")
    return aos.reshape(n, k // Q1_BLOCK_WEIGHTS, Q1_BLOCK_BYTES)


def dequantize_q1(aos: np.ndarray, n: int, k: int, rows=None) -> np.ndarray:
    """float64 ``[n, k]`` (or ``[len(rows), k]``) Q1 weights: for each position
    ``j`` take byte ``j // 8``, shift by ``j % 8``, mask one bit, map it to
    -1 / +1 and multiply by the block's decoded scale."""
    blk = _blocks_q1(aos, n, k)
    if rows is not None:
        blk = blk[np.asarray(rows)]
    qs = blk[:, :, :Q1_CODE_BYTES]
    d = f16_bits_to_float_array(blk[:, :, 16].astype(np.uint16) |
                                (blk[:, :, 17].astype(np.uint16) << 8))
    w = np.empty(qs.shape[:2] + (Q1_BLOCK_WEIGHTS,), dtype=np.float64)
    for j in range(Q1_BLOCK_WEIGHTS):
        b = (qs[:, :, j >> 3] >> (j & 7)) & 1
        w[:, :, j] = np.where(b == 1, 1.0, -1.0) * d
    return w.reshape(w.shape[0], -1)
