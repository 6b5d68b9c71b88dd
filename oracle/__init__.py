"""CPU oracle for the TQ2_0_g128 ternary matmul (test infrastructure only).

Imported by ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py``; never by the GPU library or its Python binding.
"""

from .tq2_oracle import (  # noqa: F401
    BLOCK_BYTES,
    BLOCK_WEIGHTS,
    CODE_VALUE,
    aos_bytes,
    code_of,
    dequantize,
    dequantize_block_scalar,
    dequantize_scalar,
    SILU_SLOPE_BOUND,
    error_scale,
    f16_bits_to_float,
    f16_bits_to_float_array,
    gate_up_swiglu,
    gate_up_swiglu_entries,
    gate_up_swiglu_error_scale,
    gate_up_swiglu_parts,
    matmul,
    matmul_entries,
    matmul_rows,
    matmul_scalar,
    silu,
    swiglu_from_parts,
)
from .q1_oracle import (  # noqa: F401,E402
    Q1_BLOCK_BYTES,
    Q1_BLOCK_WEIGHTS,
    bit_of,
    dequantize_block_scalar_q1,
    dequantize_q1,
    dequantize_scalar_q1,
    matmul_scalar_q1,
    q1_aos_bytes,
)
