"""gemv_tq2_g128_amd: TQ2_0_g128 ternary matmul for AMD MI355X (gfx950).

* ``csrc/``   -- the HIP kernels and the C ABI (``include/tq2.h``), built into
  ``libtq2.so`` by ``python -m gemv_tq2_g128_amd.build``;
* ``tq2``     -- the Python binding (``from gemv_tq2_g128_amd import tq2``);
  importing it raises if the library has not been built.
"""
