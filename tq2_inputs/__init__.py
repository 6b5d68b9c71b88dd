"""Seeded synthetic inputs for the TQ2_0_g128 ternary matmul.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It only draws random numbers and lays them out as the input
format; it holds none of the method's arithmetic (no code-to-value map, no
dequantisation, no products or sums).

Input format (oxibonsai-image 0.2.2, src/gpu.rs: doc of `blocks_as_bytes` and
of `ternary_matmul_gpu`): the weight of an out-major ``[N, K]`` matrix is
``N * (K / 128)`` blocks of 34 bytes each, row ``n``'s blocks contiguous and
in increasing ``k``; a block is 32 bytes of 2-bit codes followed by one
little-endian IEEE binary16 scale.

Each code byte is drawn as four independent 2-bit fields from the code
distribution.  Because the four fields are i.i.d., the byte's distribution is
the same whichever field a decoder assigns to whichever weight, so the
generator does not depend on the bit-order convention.
"""

from __future__ import annotations

import numpy as np

BLOCK_WEIGHTS = 128
BLOCK_BYTES = 34
CODE_BYTES = 32

# Code distributions, as probabilities of the 2-bit code values 0, 1, 2, 3.
# With the library's recorded convention (0 -> -1, 1 -> 0, 2 -> +1, 3 reserved)
# "uniform over {-1, 0, +1}" is equal mass on codes 0, 1, 2.
UNIFORM_TERNARY = (1.0 / 3.0, 1.0 / 3.0, 1.0 / 3.0, 0.0)
HALF_ZERO_TERNARY = (0.25, 0.5, 0.25, 0.0)


def _fields_to_byte(f0, f1, f2, f3):
    return (f0 | (f1 << 2) | (f2 << 4) | (f3 << 6)).astype(np.uint8)


# 81 base-3 digit patterns: a uniform integer in [0, 81) has four i.i.d. digits
# uniform over {0, 1, 2}.
_BASE3 = np.array([_fields_to_byte(np.uint8(v % 3), np.uint8(v // 3 % 3), np.uint8(v // 9 % 3),
                                   np.uint8(v // 27 % 3)) for v in range(81)], dtype=np.uint8)
# fields 0..3 -> codes 0, 1, 1, 2: probabilities 1/4, 1/2, 1/4
_HALF_ZERO_FIELD = np.array([0, 1, 1, 2], dtype=np.uint8)


def draw_code_bytes(rng: np.random.Generator, nbytes: int, probs) -> np.ndarray:
    """``nbytes`` bytes whose four 2-bit fields are i.i.d. with ``probs``."""
    p = np.asarray(probs, dtype=np.float64)
    p = p / p.sum()
    if np.allclose(p, UNIFORM_TERNARY):
        return _BASE3[rng.integers(0, 81, size=nbytes, dtype=np.uint8)]
    if np.allclose(p, HALF_ZERO_TERNARY):
        f = _HALF_ZERO_FIELD[rng.integers(0, 4, size=(4, nbytes), dtype=np.uint8)]
        return _fields_to_byte(f[0], f[1], f[2], f[3])
    f = rng.choice(4, size=(4, nbytes), p=p).astype(np.uint8)
    return _fields_to_byte(f[0], f[1], f[2], f[3])


def draw_scales_f16(rng: np.random.Generator, count: int, lo: float, hi: float) -> np.ndarray:
    """``count`` scales drawn U[lo, hi) and rounded to binary16 (RNE)."""
    return rng.uniform(lo, hi, size=count).astype(np.float16)


def assemble_aos(codes: np.ndarray, scales_f16: np.ndarray, n: int, k: int) -> np.ndarray:
    """Lay out code bytes ``[n*kb*32]`` and scales ``[n*kb]`` as AoS blocks."""
    kb = k // BLOCK_WEIGHTS
    blocks = np.empty((n * kb, BLOCK_BYTES), dtype=np.uint8)
    blocks[:, :CODE_BYTES] = codes.reshape(n * kb, CODE_BYTES)
    blocks[:, CODE_BYTES:] = scales_f16.astype("<f2").view(np.uint8).reshape(n * kb, 2)
    return blocks.reshape(-1)


def make_weight(rng: np.random.Generator, n: int, k: int, probs=UNIFORM_TERNARY,
                d_range=(0.01, 0.1)) -> np.ndarray:
    """A random out-major ``[n, k]`` TQ2_0_g128 weight as flat AoS bytes."""
    if k % BLOCK_WEIGHTS:
        raise ValueError("k must be a multiple of 128")
    nblk = n * (k // BLOCK_WEIGHTS)
    codes = draw_code_bytes(rng, nblk * CODE_BYTES, probs)
    scales = draw_scales_f16(rng, nblk, *d_range)
    return assemble_aos(codes, scales, n, k)


def make_activations(rng: np.random.Generator, m: int, k: int, outlier_frac: float = 0.0,
                     outlier_mult: float = 20.0) -> np.ndarray:
    """f32 ``[m, k]`` ~ N(0, 1); an i.i.d. Bernoulli(outlier_frac) mask of
    elements is multiplied by ``outlier_mult``."""
    x = rng.standard_normal((m, k), dtype=np.float32)
    if outlier_frac > 0.0:
        mask = rng.random((m, k)) < outlier_frac
        x[mask] *= np.float32(outlier_mult)
    return x


# ---------------------------------------------------------------------------
# The five workloads.  Sizes, distributions and seeds are fixed here so that
# the oracle tests, the GPU parity tests and the benchmark draw the same data.
# ---------------------------------------------------------------------------

CONFIG_SEEDS = {1: 1, 2: 2, 3: 3, 4: 4, 5: 5}

# 100-layer DiT-like chain: repeating (K, N) shapes.
CHAIN_SHAPES = ((3072, 9216), (3072, 3072), (3072, 12288), (12288, 3072))
CHAIN_LAYERS = 100
CHAIN_M = 1536
CHAIN_WEIGHT_SEED0 = 1000


def config1():
    """Ternary GEMV, M=1, K=N=1024 (8192 blocks)."""
    rng = np.random.default_rng(CONFIG_SEEDS[1])
    n = k = 1024
    w = make_weight(rng, n, k, UNIFORM_TERNARY, (0.01, 0.1))
    x = make_activations(rng, 1, k)
    return dict(name="gemv_m1_k1024_n1024", m=1, n=n, k=k, aos=w, x=x, residual=None)


def config2(with_residual: bool = False):
    """Decode GEMV, M=1, K=N=4096 (131072 blocks); optional f32 residual."""
    rng = np.random.default_rng(CONFIG_SEEDS[2])
    n = k = 4096
    w = make_weight(rng, n, k, UNIFORM_TERNARY, (0.01, 0.1))
    x = make_activations(rng, 1, k)
    r = rng.standard_normal((1, n), dtype=np.float32)
    return dict(name="gemv_m1_k4096_n4096" + ("_residual" if with_residual else ""),
                m=1, n=n, k=k, aos=w, x=x, residual=r if with_residual else None)


def config3(m: int):
    """Small-batch prefill GEMM, K=4096, N=11008, 50% zero codes."""
    if m not in (7, 8, 9, 100):
        raise ValueError("config 3 is defined for M in {7, 8, 9, 100}")
    rng = np.random.default_rng(CONFIG_SEEDS[3])
    n, k = 11008, 4096
    w = make_weight(rng, n, k, HALF_ZERO_TERNARY, (0.005, 0.05))
    xs = make_activations(rng, 100, k)
    return dict(name=f"gemm_m{m}_k4096_n11008", m=m, n=n, k=k, aos=w,
                x=np.ascontiguousarray(xs[:m]), residual=None)


def config4():
    """Large-M DiT-shaped GEMM, M=1536, K=N=3072, 1% outliers x20."""
    rng = np.random.default_rng(CONFIG_SEEDS[4])
    m, n, k = 1536, 3072, 3072
    w = make_weight(rng, n, k, UNIFORM_TERNARY, (0.01, 0.1))
    x = make_activations(rng, m, k, outlier_frac=0.01, outlier_mult=20.0)
    return dict(name="gemm_m1536_k3072_n3072", m=m, n=n, k=k, aos=w, x=x, residual=None)


def chain_layer_shape(layer: int):
    return CHAIN_SHAPES[layer % len(CHAIN_SHAPES)]


def chain_layer_weight(layer: int) -> np.ndarray:
    """Weights of layer ``layer`` of the 100-layer chain (config-4 distributions)."""
    k, n = chain_layer_shape(layer)
    rng = np.random.default_rng(CHAIN_WEIGHT_SEED0 + layer)
    return make_weight(rng, n, k, UNIFORM_TERNARY, (0.01, 0.1))


def chain_input() -> np.ndarray:
    rng = np.random.default_rng(CONFIG_SEEDS[5])
    return make_activations(rng, CHAIN_M, CHAIN_SHAPES[0][0])


def random_case(seed: int, m: int, n: int, k: int, probs=UNIFORM_TERNARY,
                d_range=(0.01, 0.1), residual: bool = False, outlier_frac: float = 0.0):
    """A generic seeded case for shape sweeps and edge cases."""
    rng = np.random.default_rng(seed)
    w = make_weight(rng, n, k, probs, d_range)
    x = make_activations(rng, m, k, outlier_frac=outlier_frac)
    r = rng.standard_normal((m, n), dtype=np.float32) if residual else None
    return dict(name=f"case_s{seed}_m{m}_n{n}_k{k}", m=m, n=n, k=k, aos=w, x=x, residual=r)


def swiglu_case(seed: int, m: int, n: int, k: int, probs=HALF_ZERO_TERNARY,
                d_range=(0.005, 0.05), outlier_frac: float = 0.0):
    """Gate and up weights (both ``[n, k]``) and activations ``[m, k]`` for the
    fused gate/up + SwiGLU op; defaults follow the prefill GEMM workload's
    code and scale distributions."""
    rng = np.random.default_rng(seed)
    gate = make_weight(rng, n, k, probs, d_range)
    up = make_weight(rng, n, k, probs, d_range)
    x = make_activations(rng, m, k, outlier_frac=outlier_frac)
    return dict(name=f"swiglu_s{seed}_m{m}_n{n}_k{k}", m=m, n=n, k=k, gate=gate, up=up, x=x)


# Feed-forward gate/up workload: K = 4096 -> N = 11008 (the prefill GEMM
# workload's projection shape), half-zero codes, d ~ U[0.005, 0.05].
SWIGLU_K, SWIGLU_N = 4096, 11008
SWIGLU_WEIGHT_SEED = 33


def swiglu_weights():
    """Gate and up weights of the feed-forward workload (AoS bytes)."""
    rng = np.random.default_rng(SWIGLU_WEIGHT_SEED)
    gate = make_weight(rng, SWIGLU_N, SWIGLU_K, HALF_ZERO_TERNARY, (0.005, 0.05))
    up = make_weight(rng, SWIGLU_N, SWIGLU_K, HALF_ZERO_TERNARY, (0.005, 0.05))
    return gate, up


def swiglu_activations(m: int) -> np.ndarray:
    """``m`` activation rows of the feed-forward workload, x ~ N(0, 1)."""
    return make_activations(np.random.default_rng(SWIGLU_WEIGHT_SEED + 1 + m), m, SWIGLU_K)


def swiglu_workload(m: int):
    """Gate/up weights of the feed-forward workload and ``m`` activation rows."""
    gate, up = swiglu_weights()
    return dict(name=f"swiglu_m{m}_k{SWIGLU_K}_n{SWIGLU_N}", m=m, n=SWIGLU_N, k=SWIGLU_K,
                gate=gate, up=up, x=swiglu_activations(m))


# ---------------------------------------------------------------------------
# Q1_g128 (1-bit sibling format): blocks of 128 weights, 16 bytes of bits then
# a little-endian binary16 scale (18 bytes).  Bits are drawn i.i.d. fair, so
# the draw does not depend on the bit-order convention either.
# ---------------------------------------------------------------------------

Q1_BLOCK_BYTES = 18
Q1_CODE_BYTES = 16


def make_weight_q1(rng: np.random.Generator, n: int, k: int,
                   d_range=(0.01, 0.1)) -> np.ndarray:
    """A random out-major ``[n, k]`` Q1_g128 weight as flat AoS bytes."""
    if k % BLOCK_WEIGHTS:
        raise ValueError("k must be a multiple of 128")
    nblk = n * (k // BLOCK_WEIGHTS)
    bits = rng.integers(0, 256, size=nblk * Q1_CODE_BYTES, dtype=np.uint8)
    scales = draw_scales_f16(rng, nblk, *d_range)
    blocks = np.empty((nblk, Q1_BLOCK_BYTES), dtype=np.uint8)
    blocks[:, :Q1_CODE_BYTES] = bits.reshape(nblk, Q1_CODE_BYTES)
    blocks[:, Q1_CODE_BYTES:] = scales.astype("<f2").view(np.uint8).reshape(nblk, 2)
    return blocks.reshape(-1)


def random_case_q1(seed: int, m: int, n: int, k: int, d_range=(0.01, 0.1),
                   residual: bool = False, outlier_frac: float = 0.0):
    """A generic seeded Q1_g128 case for shape sweeps and edge cases."""
    rng = np.random.default_rng(seed)
    w = make_weight_q1(rng, n, k, d_range)
    x = make_activations(rng, m, k, outlier_frac=outlier_frac)
    r = rng.standard_normal((m, n), dtype=np.float32) if residual else None
    return dict(name=f"q1_s{seed}_m{m}_n{n}_k{k}", m=m, n=n, k=k, aos=w, x=x, residual=r)


Q1_SEEDS = {"decode": 21, "gemm": 24}


def q1_decode(with_residual: bool = True):
    """Q1 decode GEMV, M=1, K=N=4096 (131072 blocks, 2.36 MB), d ~ U[0.01, 0.1]."""
    rng = np.random.default_rng(Q1_SEEDS["decode"])
    n = k = 4096
    w = make_weight_q1(rng, n, k, (0.01, 0.1))
    x = make_activations(rng, 1, k)
    r = rng.standard_normal((1, n), dtype=np.float32)
    return dict(name="q1_gemv_m1_k4096_n4096" + ("_residual" if with_residual else ""),
                m=1, n=n, k=k, aos=w, x=x, residual=r if with_residual else None)


def q1_gemm():
    """Q1 large-M GEMM, M=1536, K=N=3072, x ~ N(0, 1) with 1% outliers x20."""
    rng = np.random.default_rng(Q1_SEEDS["gemm"])
    m, n, k = 1536, 3072, 3072
    w = make_weight_q1(rng, n, k, (0.01, 0.1))
    x = make_activations(rng, m, k, outlier_frac=0.01, outlier_mult=20.0)
    return dict(name="q1_gemm_m1536_k3072_n3072", m=m, n=n, k=k, aos=w, x=x, residual=None)


def swiglu_case_q1(seed: int, m: int, n: int, k: int, d_range=(0.005, 0.05)):
    """Q1 gate and up weights (both ``[n, k]``) and activations ``[m, k]``."""
    rng = np.random.default_rng(seed)
    gate = make_weight_q1(rng, n, k, d_range)
    up = make_weight_q1(rng, n, k, d_range)
    x = make_activations(rng, m, k)
    return dict(name=f"q1_swiglu_s{seed}_m{m}_n{n}_k{k}", m=m, n=n, k=k, gate=gate, up=up, x=x)
