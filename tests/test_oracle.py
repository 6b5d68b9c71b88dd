"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here runs on the CPU.  The checks are written as functions of the
oracle's ``dequantize`` / ``matmul`` so that ``test_pins_catch_planted_mistakes``
can run them against deliberately broken copies of the oracle (planted on the
CPU) and show that each plausible mistake fails at least one pin.

Sources: oxibonsai-image 0.2.2, src/gpu.rs (module doc "Correctness contract";
doc of ``blocks_as_bytes``; doc of ``ternary_matmul_gpu``; its unit tests).
The bit order (least significant 2-bit field first) and the code map
(0 -> -1, 1 -> 0, 2 -> +1, 3 -> 0) are the recorded convention: the pages
print neither, so the hand-worked cases below pin the oracle to that
convention, not to a printed example.
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import tq2_oracle as O
import tq2_inputs as G

ONE = 0x3C00        # binary16 1.0
HALF_NEG = 0xB800   # binary16 -0.5


def block(qs_bytes, d_bits):
    qs = bytes(qs_bytes)
    assert len(qs) == 32
    return qs + bytes([d_bits & 0xFF, (d_bits >> 8) & 0xFF])


# ---------------------------------------------------------------------------
# binary16
# ---------------------------------------------------------------------------

def test_f16_decoder_exhaustive_against_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.f16_bits_to_float_array(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_f16_scalar_decoder_exhaustive_against_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    for b in range(65536):
        g = oracle.f16_bits_to_float(b)
        r = ref[b]
        if np.isnan(r):
            assert g != g
        else:
            assert g == r and np.signbit(g) == np.signbit(r), b


# ---------------------------------------------------------------------------
# Pins, as functions of (dequantize, matmul).
# ---------------------------------------------------------------------------

def pin_hand_worked_first_byte(deq):
    # qs[0] = 0x02 -> fields (LSB first) 2, 0, 0, 0 -> +1, -1, -1, -1; rest 0x55
    # (every field 1 -> 0); d = 1.0.
    b = block([0x02] + [0x55] * 31, ONE)
    w = deq(np.frombuffer(b, np.uint8), 1, 128)[0]
    want = np.zeros(128)
    want[0], want[1], want[2], want[3] = 1.0, -1.0, -1.0, -1.0
    return np.array_equal(w, want)


def pin_hand_worked_last_byte(deq):
    # qs[31] = 0x24 = 0b00_10_01_00 -> weights 124..127 have codes 0, 1, 2, 0
    # -> -1, 0, +1, -1; times d = -0.5 -> +0.5, 0, -0.5, +0.5.
    b = block([0x55] * 31 + [0x24], HALF_NEG)
    w = deq(np.frombuffer(b, np.uint8), 1, 128)[0]
    want = np.zeros(128)
    want[124], want[125], want[126], want[127] = 0.5, 0.0, -0.5, 0.5
    return np.array_equal(w, want)


def pin_code3_is_zero(deq):
    b = block([0xFF] * 32, ONE)
    return np.array_equal(deq(np.frombuffer(b, np.uint8), 1, 128)[0], np.zeros(128))


def pin_two_block_row(mm):
    # Row of two blocks (K = 256).  Block 0: qs[1] = 0x09 = 0b00_00_10_01 ->
    # weights 4..7 = codes 1, 2, 0, 0 -> 0, +1, -1, -1, rest 0, d = 2.0 (0x4000).
    # Block 1: qs[0] = 0x06 = 0b00_00_01_10 -> weights 128..131 = codes 2, 1, 0, 0
    # -> +1, 0, -1, -1, rest 0, d = 0.25 (0x3400).
    # x[k] = k + 1:  2*(x5 - x6 - x7) + 0.25*(x128 - x130 - x131)
    #             = 2*(6 - 7 - 8) + 0.25*(129 - 131 - 132) = -18 - 33.5 = -51.5
    b0 = block([0x55, 0x09] + [0x55] * 30, 0x4000)
    b1 = block([0x06] + [0x55] * 31, 0x3400)
    aos = np.frombuffer(b0 + b1, np.uint8)
    x = (np.arange(256, dtype=np.float32) + 1.0)[None, :]
    return float(mm(aos, x, 1, 256)[0, 0]) == -51.5


def pin_unit_vectors_read_back_every_weight(deq):
    # Brute force over every (position, code) pair: one block per code value
    # with that code at every position, and one block per position with code 2
    # there and code 1 elsewhere.  Positions are located with numpy's
    # little-endian bit unpacking of the 256-bit qs string, a route independent
    # of the oracle's shift-and-mask.
    ok = True
    for c in range(4):
        byte = c | (c << 2) | (c << 4) | (c << 6)
        w = deq(np.frombuffer(block([byte] * 32, ONE), np.uint8), 1, 128)[0]
        ok &= np.array_equal(w, np.full(128, O.CODE_VALUE[c]))
    for j in range(128):
        bits = np.zeros(256, dtype=np.uint8)
        bits[0::2] = 1                       # code 1 (value 0) everywhere
        bits[2 * j], bits[2 * j + 1] = 0, 1  # code 2 at position j
        qs = np.packbits(bits, bitorder="little")
        w = deq(np.frombuffer(block(qs.tolist(), ONE), np.uint8), 1, 128)[0]
        want = np.zeros(128)
        want[j] = 1.0
        ok &= np.array_equal(w, want)
    return bool(ok)


def _rand_case(seed, m, n, k, probs=G.UNIFORM_TERNARY):
    c = G.random_case(seed, m, n, k, probs=probs, residual=True)
    return c["aos"], c["x"], c["residual"]


def _replace_codes(aos, n, k, byte_value=None, byte_map=None):
    a = aos.reshape(-1, 34).copy()
    if byte_value is not None:
        a[:, :32] = byte_value
    if byte_map is not None:
        a[:, :32] = byte_map[a[:, :32]]
    return a.reshape(-1)


def _scales(aos, n, k):
    a = aos.reshape(n, k // 128, 34)
    bits = a[:, :, 32].astype(np.uint16) | (a[:, :, 33].astype(np.uint16) << 8)
    return bits.view(np.float16).astype(np.float64)          # numpy's decoder


def pin_closed_forms(mm):
    aos, x, _ = _rand_case(11, 3, 5, 384)
    n, k = 5, 384
    d = _scales(aos, n, k)                                     # [n, kb]
    blocksum = x.astype(np.float64).reshape(3, k // 128, 128).sum(axis=2)   # [m, kb]
    plus = blocksum @ d.T                                       # every weight = +d
    ok = True
    ok &= np.array_equal(mm(_replace_codes(aos, n, k, 0x55), x, n, k), np.zeros((3, n)))
    ok &= np.allclose(mm(_replace_codes(aos, n, k, 0xAA), x, n, k), plus, rtol=1e-13, atol=0)
    ok &= np.allclose(mm(_replace_codes(aos, n, k, 0x00), x, n, k), -plus, rtol=1e-13, atol=0)
    zero_d = aos.reshape(-1, 34).copy()
    zero_d[:, 32:] = 0
    ok &= np.array_equal(mm(zero_d.reshape(-1), x, n, k), np.zeros((3, n)))
    return bool(ok)


def _swap02_table():
    t = np.zeros(256, dtype=np.uint8)
    for b in range(256):
        out = 0
        for f in range(4):
            c = (b >> (2 * f)) & 3
            c = {0: 2, 2: 0}.get(c, c)
            out |= c << (2 * f)
        t[b] = out
    return t


def pin_symmetries(mm):
    n, k = 7, 256
    aos, x, r = _rand_case(12, 4, n, k)
    base = mm(aos, x, n, k)
    ok = True
    # swapping codes 0 <-> 2 negates every weight
    ok &= np.allclose(mm(_replace_codes(aos, n, k, byte_map=_swap02_table()), x, n, k),
                      -base, rtol=1e-13, atol=1e-13)
    # doubling every scale (exponent + 1, no overflow at these magnitudes) doubles out
    a = aos.reshape(-1, 34).copy()
    bits = a[:, 32].astype(np.uint16) | (a[:, 33].astype(np.uint16) << 8)
    bits = bits + (1 << 10)
    a[:, 32] = bits & 0xFF
    a[:, 33] = bits >> 8
    ok &= np.array_equal(mm(a.reshape(-1), x, n, k), 2.0 * base)
    # residual is added once
    ok &= np.allclose(mm(aos, x, n, k, r) - base, r.astype(np.float64), rtol=0, atol=1e-12)
    # linearity in x
    y = np.random.default_rng(5).standard_normal(x.shape).astype(np.float32)
    lhs = mm(aos, 2.0 * x.astype(np.float64) - 3.0 * y.astype(np.float64), n, k)
    ok &= np.allclose(lhs, 2.0 * base - 3.0 * mm(aos, y, n, k), rtol=1e-12, atol=1e-12)
    # row permutation of W permutes the output columns
    perm = np.array([3, 0, 6, 1, 5, 2, 4])
    ap = aos.reshape(n, -1)[perm].reshape(-1)
    ok &= np.array_equal(mm(ap, x, n, k), base[:, perm])
    # splitting K into two halves sums the outputs
    h = k // 2
    wa = aos.reshape(n, k // 128, 34)
    lo = np.ascontiguousarray(wa[:, : h // 128]).reshape(-1)
    hi = np.ascontiguousarray(wa[:, h // 128:]).reshape(-1)
    ok &= np.allclose(mm(lo, x[:, :h], n, h) + mm(hi, x[:, h:], n, h), base,
                      rtol=1e-12, atol=1e-12)
    return bool(ok)


def pin_against_scalar_triple_loop(mm):
    ok = True
    for seed, (m, n, k) in enumerate([(1, 1, 128), (2, 3, 256), (3, 2, 384), (1, 4, 128)]):
        aos, x, r = _rand_case(100 + seed, m, n, k)
        ref = np.array(O.matmul_scalar(bytes(aos), x.tolist(), n, k, r.tolist()))
        ok &= np.allclose(mm(aos, x, n, k, r), ref, rtol=1e-12, atol=1e-12)
    return bool(ok)


def pin_zero_blocks_from_pages(deq, golden):
    nb = golden["blocks"]
    raw = block([golden["qs_byte"]] * 32, golden["d_bits"]) * nb
    ok = len(raw) == golden["total_bytes"] == nb * golden["block_bytes"]
    ok &= O.aos_bytes(1, 128 * nb) == golden["total_bytes"]
    ok &= O.aos_bytes(nb, 128) == golden["total_bytes"]
    w = deq(np.frombuffer(raw, np.uint8), 1, 128 * nb)
    ok &= np.array_equal(w, np.full((1, 128 * nb), golden["expected_output"]))
    return bool(ok)


# ---------------------------------------------------------------------------
# The tests.
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def golden(golden_dir):
    with open(os.path.join(golden_dir, "zero_blocks.json")) as f:
        return json.load(f)


def test_zero_blocks_from_pages(golden):
    assert pin_zero_blocks_from_pages(O.dequantize, golden)


def test_block_is_34_bytes():
    assert O.BLOCK_BYTES == 34 and O.aos_bytes(1, 128) == 34
    assert O.aos_bytes(4096, 4096) == 131072 * 34            # 4,456,448 B


def test_hand_worked_blocks():
    assert pin_hand_worked_first_byte(O.dequantize)
    assert pin_hand_worked_last_byte(O.dequantize)
    assert pin_code3_is_zero(O.dequantize)


def test_hand_worked_blocks_scalar():
    def deq_scalar(aos, n, k):
        return np.array(O.dequantize_scalar(bytes(aos), n, k))
    assert pin_hand_worked_first_byte(deq_scalar)
    assert pin_hand_worked_last_byte(deq_scalar)
    assert pin_code3_is_zero(deq_scalar)
    assert pin_unit_vectors_read_back_every_weight(deq_scalar)


def test_two_block_row():
    assert pin_two_block_row(O.matmul)


def test_unit_vectors_read_back_every_weight():
    assert pin_unit_vectors_read_back_every_weight(O.dequantize)


def test_closed_forms():
    assert pin_closed_forms(O.matmul)


def test_symmetries_and_invariants():
    assert pin_symmetries(O.matmul)


def test_numpy_oracle_matches_scalar_triple_loop():
    assert pin_against_scalar_triple_loop(O.matmul)


def test_special_scales():
    # subnormal, negative zero and negative scales decode exactly
    for d_bits, d in [(0x0001, 2.0 ** -24), (0x8000, -0.0), (0xB800, -0.5), (0x7BFF, 65504.0)]:
        w = O.dequantize(np.frombuffer(block([0xAA] * 32, d_bits), np.uint8), 1, 128)[0]
        assert np.array_equal(w, np.full(128, d))


def test_entries_and_rows_match_full():
    n, k = 9, 512
    aos, x, r = _rand_case(21, 5, n, k)
    full = O.matmul(aos, x, n, k, r)
    s_full = O.error_scale(aos, x, n, k, r)
    rows = np.array([0, 4, 2, 2])
    cols = np.array([8, 0, 3, 3])
    ref, s = O.matmul_entries(aos, x, n, k, rows, cols, r)
    assert np.allclose(ref, full[rows, cols], rtol=1e-13, atol=1e-13)
    assert np.allclose(s, s_full[rows, cols], rtol=1e-13)
    ref2, s2 = O.matmul_rows(aos, x, n, k, [1, 7], r)
    assert np.allclose(ref2, full[:, [1, 7]], rtol=1e-13, atol=1e-13)
    assert np.allclose(s2, s_full[:, [1, 7]], rtol=1e-13)


def test_error_scale_bounds_result():
    n, k = 6, 384
    aos, x, r = _rand_case(22, 3, n, k)
    ref = O.matmul(aos, x, n, k, r)
    s = O.error_scale(aos, x, n, k, r)
    assert np.all(np.abs(ref) <= s * (1 + 1e-12))
    w = np.array(O.dequantize_scalar(bytes(aos), n, k))
    brute = np.abs(x.astype(np.float64))[:, None, :] * np.abs(w)[None, :, :]
    assert np.allclose(s, brute.sum(axis=2) + np.abs(r), rtol=1e-13)


def test_length_and_shape_errors():
    with pytest.raises(ValueError):
        O.dequantize(np.zeros(33, np.uint8), 1, 128)
    with pytest.raises(ValueError):
        O.dequantize(np.zeros(34, np.uint8), 1, 100)


def test_generator_distributions():
    # the generator draws what the workloads name (checked through the oracle's
    # decode): codes uniform over {-1, 0, +1}, or half zeros; scales in range.
    n, k = 64, 1024
    w = O.dequantize(G.make_weight(np.random.default_rng(0), n, k), n, k)
    sign = np.sign(w)
    for v in (-1, 0, 1):
        assert abs(np.mean(sign == v) - 1 / 3) < 0.01
    d = np.abs(w[w != 0])
    assert d.min() >= 0.0099 and d.max() <= 0.1001
    w2 = O.dequantize(G.make_weight(np.random.default_rng(1), n, k, G.HALF_ZERO_TERNARY,
                                    (0.005, 0.05)), n, k)
    assert abs(np.mean(w2 == 0) - 0.5) < 0.01
    assert abs(np.mean(w2 > 0) - 0.25) < 0.01


# ---------------------------------------------------------------------------
# Planted mistakes: each broken copy of the oracle must fail some pin.
# ---------------------------------------------------------------------------

def _mutant_dequantize(kind):
    def deq(aos, n, k, rows=None):
        blk = O._blocks(aos, n, k)
        qs = blk[:, :, :32]
        d_bits = blk[:, :, 32].astype(np.uint16) | (blk[:, :, 33].astype(np.uint16) << 8)
        if kind == "scale_big_endian":
            d_bits = blk[:, :, 33].astype(np.uint16) | (blk[:, :, 32].astype(np.uint16) << 8)
        d = O.f16_bits_to_float_array(d_bits)
        vals = {"code_map_swapped": [1.0, 0.0, -1.0, 0.0],
                "code3_is_one": [-1.0, 0.0, 1.0, 1.0],
                "zero_is_code0": [0.0, -1.0, 1.0, 0.0]}.get(kind, [-1.0, 0.0, 1.0, 0.0])
        vals = np.array(vals)
        w = np.empty(qs.shape[:2] + (128,))
        for j in range(128):
            if kind == "msb_first":
                c = (qs[:, :, j >> 2] >> (6 - 2 * (j & 3))) & 3
            elif kind == "strided":
                c = (qs[:, :, j & 31] >> (2 * (j >> 5))) & 3
            else:
                c = (qs[:, :, j >> 2] >> (2 * (j & 3))) & 3
            w[:, :, j] = vals[c] * (1.0 if kind == "scale_dropped" else d)
        return w.reshape(w.shape[0], -1)
    return deq


def _mutant_matmul(kind, deq=None):
    deq = deq or O.dequantize

    def mm(aos, x, n, k, residual=None):
        x64 = np.asarray(x, np.float64).reshape(-1, k)
        w = deq(aos, n, k)
        if kind == "dropped_last_block":
            w = w.copy()
            w[:, -128:] = 0
        if kind == "reversed_k":
            w = w[:, ::-1]
        out = x64 @ w.T
        if residual is not None and kind != "residual_dropped":
            out = np.asarray(residual, np.float64).reshape(out.shape) + out
        return out
    return mm


@pytest.mark.parametrize("kind", ["msb_first", "strided", "code_map_swapped", "code3_is_one",
                                  "zero_is_code0", "scale_dropped", "scale_big_endian"])
def test_pins_catch_planted_decode_mistakes(kind):
    deq = _mutant_dequantize(kind)
    mm = _mutant_matmul("none", deq)
    results = [pin_hand_worked_first_byte(deq), pin_hand_worked_last_byte(deq),
               pin_code3_is_zero(deq), pin_unit_vectors_read_back_every_weight(deq),
               pin_two_block_row(mm), pin_closed_forms(mm), pin_symmetries(mm)]
    assert not all(results), kind


@pytest.mark.parametrize("kind", ["dropped_last_block", "reversed_k", "residual_dropped"])
def test_pins_catch_planted_sum_mistakes(kind):
    mm = _mutant_matmul(kind)
    results = [pin_two_block_row(mm), pin_closed_forms(mm), pin_symmetries(mm),
               pin_against_scalar_triple_loop(mm)]
    assert not all(results), kind


# ---------------------------------------------------------------------------
# SiLU and the fused gate/up + SwiGLU composition (the ternary counterpart of
# the fused_gate_up_swiglu_q1 / fused_gate_up_swiglu_gemm_q1 pipelines of
# oxibonsai-kernels 0.1.5, pipelines.rs).  SiLU(z) = z * logistic(z); the pins
# use the logistic function's textbook values, SciPy's expit as an
# independent library route, and the identity silu(z) - silu(-z) = z.
# ---------------------------------------------------------------------------

from scipy.special import expit  # noqa: E402

LOGISTIC_1 = 0.7310585786300049      # 1 / (1 + e^-1)
LOGISTIC_2 = 0.8807970779778823      # 1 / (1 + e^-2)


def pin_silu_values(silu):
    z = np.linspace(-30.0, 30.0, 6001)
    ok = float(silu(0.0)) == 0.0
    ok &= abs(float(silu(1.0)) - LOGISTIC_1) <= 2e-16
    ok &= abs(float(silu(-1.0)) - (LOGISTIC_1 - 1.0)) <= 2e-16
    ok &= abs(float(silu(2.0)) - 2.0 * LOGISTIC_2) <= 4e-16
    ok &= np.allclose(silu(z), z * expit(z), rtol=1e-14, atol=1e-300)
    ok &= np.allclose(silu(z) - silu(-z), z, rtol=0, atol=1e-13)
    big = silu(np.array([800.0, -800.0]))
    ok &= bool(np.all(np.isfinite(big))) and big[0] == 800.0 and big[1] == 0.0
    # the slope bound used by the error scale holds and is nearly tight
    zz = np.linspace(-20.0, 20.0, 400001)
    slope = np.diff(silu(zz)) / np.diff(zz)
    ok &= slope.max() < O.SILU_SLOPE_BOUND and slope.max() > 1.09 and slope.min() > -0.11
    return bool(ok)


def pin_swiglu_hand_worked(sw):
    # One row x = 1 (K = 128).  Gate: every code 2 (+1), d = 2^-6 -> g = 2.
    # Up: every code 0 (-1), d = 0.5 -> u = -64.  out = silu(2) * (-64)
    # = -128 * logistic(2).
    gate = np.frombuffer(block([0xAA] * 32, 0x2400), np.uint8)
    up = np.frombuffer(block([0x00] * 32, 0x3800), np.uint8)
    x = np.ones((1, 128), np.float32)
    return abs(float(sw(gate, up, x, 1, 128)[0, 0]) + 128.0 * LOGISTIC_2) <= 1e-12


def pin_swiglu_structure(sw):
    n, k = 6, 384
    c = G.swiglu_case(41, 3, n, k)
    gate, up, x = c["gate"], c["up"], c["x"]
    base = sw(gate, up, x, n, k)
    ok = True
    # a zero gate or a zero up projection gives zero
    ok &= np.array_equal(sw(_replace_codes(gate, n, k, 0x55), up, x, n, k), np.zeros((3, n)))
    ok &= np.array_equal(sw(gate, _replace_codes(up, n, k, 0x55), x, n, k), np.zeros((3, n)))
    # negating the up weight negates the output; negating the gate does not
    neg = _swap02_table()
    ok &= np.allclose(sw(gate, _replace_codes(up, n, k, byte_map=neg), x, n, k), -base,
                      rtol=1e-13, atol=1e-15)
    ok &= not np.allclose(sw(_replace_codes(gate, n, k, byte_map=neg), up, x, n, k), -base,
                          rtol=1e-6, atol=1e-9)
    # gate == up: out = u^2 logistic(u) >= 0
    ok &= bool(np.all(sw(up, up, x, n, k) >= 0))
    # a row permutation applied to both weights permutes the output columns
    perm = np.array([4, 0, 5, 1, 3, 2])
    gp = gate.reshape(n, -1)[perm].reshape(-1)
    upp = up.reshape(n, -1)[perm].reshape(-1)
    ok &= np.array_equal(sw(gp, upp, x, n, k), base[:, perm])
    # against the scalar triple loop and SciPy's logistic function
    gs = np.array(O.matmul_scalar(bytes(gate), x.tolist(), n, k))
    us = np.array(O.matmul_scalar(bytes(up), x.tolist(), n, k))
    ok &= np.allclose(base, gs * expit(gs) * us, rtol=1e-12, atol=1e-15)
    return bool(ok)


def test_silu_values():
    assert pin_silu_values(O.silu)


def test_swiglu_hand_worked():
    assert pin_swiglu_hand_worked(O.gate_up_swiglu)


def test_swiglu_structure():
    assert pin_swiglu_structure(O.gate_up_swiglu)


def test_swiglu_error_scale_bounds_perturbations():
    # Projections moved by up to tol * sum_k |x w| (every sign pattern, plus
    # random points inside the box) move the output by at most tol * E.
    n, k = 8, 512
    c = G.swiglu_case(42, 4, n, k, probs=G.UNIFORM_TERNARY, d_range=(0.05, 0.5))
    gate, up, x = c["gate"], c["up"], c["x"]
    g, u = O.matmul(gate, x, n, k), O.matmul(up, x, n, k)
    sg, su = O.error_scale(gate, x, n, k), O.error_scale(up, x, n, k)
    ref = O.gate_up_swiglu(gate, up, x, n, k)
    rng = np.random.default_rng(7)
    for tol in (1e-5, 2e-3, 0.05):
        e = O.gate_up_swiglu_error_scale(gate, up, x, n, k, tol)
        trials = [(a, b) for a in (-1.0, 1.0) for b in (-1.0, 1.0)]
        trials += [tuple(rng.uniform(-1, 1, size=(2,) + g.shape)) for _ in range(20)]
        for a, b in trials:
            moved = O.silu(g + a * tol * sg) * (u + b * tol * su)
            assert np.all(np.abs(moved - ref) <= tol * e * (1 + 1e-12) + 1e-300)
    # and it is not loose by orders of magnitude where the gate is steep
    e = O.gate_up_swiglu_error_scale(gate, up, x, n, k, 2e-3)
    moved = O.silu(g + 2e-3 * sg) * u
    assert np.max(np.abs(moved - ref) / (2e-3 * e)) > 0.2


def test_swiglu_entries_match_full():
    n, k = 9, 256
    c = G.swiglu_case(43, 5, n, k)
    full = O.gate_up_swiglu(c["gate"], c["up"], c["x"], n, k)
    e_full = O.gate_up_swiglu_error_scale(c["gate"], c["up"], c["x"], n, k, 1e-5)
    rows, cols = np.array([0, 4, 2]), np.array([8, 0, 3])
    ref, e = O.gate_up_swiglu_entries(c["gate"], c["up"], c["x"], n, k, rows, cols, 1e-5)
    assert np.allclose(ref, full[rows, cols], rtol=1e-13, atol=1e-15)
    assert np.allclose(e, e_full[rows, cols], rtol=1e-13)


def test_swiglu_parts_match_plain_route():
    n, k = 7, 384
    c = G.swiglu_case(44, 3, n, k)
    parts = O.gate_up_swiglu_parts(c["gate"], c["up"], c["x"], n, k)
    for tol in (1e-5, 2e-3):
        ref, e = O.swiglu_from_parts(parts, tol)
        assert np.allclose(ref, O.gate_up_swiglu(c["gate"], c["up"], c["x"], n, k),
                           rtol=1e-13, atol=1e-15)
        assert np.allclose(e, O.gate_up_swiglu_error_scale(c["gate"], c["up"], c["x"], n, k, tol),
                           rtol=1e-13)


def _mutant_swiglu(kind):
    def silu(z):
        z = np.asarray(z, np.float64)
        if kind == "sigmoid":
            return expit(z)
        if kind == "exp_sign":
            return z / (1.0 + np.exp(np.minimum(z, 700)))
        if kind == "relu":
            return np.maximum(z, 0.0)
        return O.silu(z)

    def sw(gate, up, x, n, k):
        g = O.matmul(gate, x, n, k)
        u = O.matmul(up, x, n, k)
        if kind == "swapped":
            g, u = u, g
        if kind == "sum":
            return silu(g) + u
        if kind == "gate_only":
            return silu(g)
        return silu(g) * u
    return silu, sw


@pytest.mark.parametrize("kind", ["sigmoid", "exp_sign", "relu", "swapped", "sum", "gate_only"])
def test_pins_catch_planted_swiglu_mistakes(kind):
    silu, sw = _mutant_swiglu(kind)
    results = [pin_silu_values(silu), pin_swiglu_hand_worked(sw), pin_swiglu_structure(sw)]
    assert not all(results), kind


# ---------------------------------------------------------------------------
# Q1_g128 (1-bit sibling format).  The pages name the q1 kernels but print no
# layout; the pins hold the oracle to the recorded convention (18-byte block:
# qs[16] then a little-endian binary16 d; bit j = (qs[j // 8] >> (j % 8)) & 1;
# set -> +d, clear -> -d).
# ---------------------------------------------------------------------------

from oracle import q1_oracle as Q  # noqa: E402


def q1_block(qs_bytes, d_bits):
    qs = bytes(qs_bytes)
    assert len(qs) == 16
    return qs + bytes([d_bits & 0xFF, (d_bits >> 8) & 0xFF])


def _q1(b):
    return np.frombuffer(b, np.uint8)


def pin_q1_hand_worked(deq):
    # qs[0] = 0x05 -> bits 1, 0, 1, 0, 0, 0, 0, 0 (LSB first); every other bit
    # clear; d = 0.5 -> +0.5, -0.5, +0.5, then -0.5 for weights 3..127.
    w = deq(_q1(q1_block([0x05] + [0x00] * 15, 0x3800)), 1, 128)[0]
    want = np.full(128, -0.5)
    want[0] = want[2] = 0.5
    ok = np.array_equal(w, want)
    # qs[15] = 0x7F, every other byte 0xFF; d = -2 -> -2 everywhere except
    # weight 127 (bit 7 of byte 15, clear) = +2.
    w = deq(_q1(q1_block([0xFF] * 15 + [0x7F], 0xC000)), 1, 128)[0]
    want = np.full(128, -2.0)
    want[127] = 2.0
    ok &= np.array_equal(w, want)
    return bool(ok)


def pin_q1_unit_vectors(deq):
    # One block per position j with only bit j set (numpy's little-endian
    # bit packing locates it, independent of the oracle's shift-and-mask).
    ok = True
    for j in range(128):
        bits = np.zeros(128, dtype=np.uint8)
        bits[j] = 1
        qs = np.packbits(bits, bitorder="little")
        w = deq(_q1(q1_block(qs.tolist(), ONE)), 1, 128)[0]
        want = np.full(128, -1.0)
        want[j] = 1.0
        ok &= np.array_equal(w, want)
    return bool(ok)


def pin_q1_two_block_row(mm):
    # x[k] = k + 1 (K = 256).  Block 0: d = 1, every bit set but weight 0:
    # 8256 - 2 * 1 = 8254.  Block 1: d = 0.25, every bit clear but weight 127
    # (k = 255): 0.25 * (-24640 + 2 * 256) = -6032.  Total 2222.
    b0 = q1_block([0xFE] + [0xFF] * 15, ONE)
    b1 = q1_block([0x00] * 15 + [0x80], 0x3400)
    x = (np.arange(256, dtype=np.float32) + 1.0)[None, :]
    return float(mm(_q1(b0 + b1), x, 1, 256)[0, 0]) == 2222.0


def pin_q1_closed_forms(mm):
    n, k = 5, 384
    c = G.random_case_q1(31, 3, n, k)
    aos, x = c["aos"], c["x"]
    a = aos.reshape(n, k // 128, 18)
    d = (a[:, :, 16].astype(np.uint16) | (a[:, :, 17].astype(np.uint16) << 8)).view(
        np.float16).astype(np.float64)
    blocksum = x.astype(np.float64).reshape(3, k // 128, 128).sum(axis=2)
    plus = blocksum @ d.T

    def with_bits(v):
        b = a.copy()
        b[:, :, :16] = v
        return b.reshape(-1)
    ok = np.allclose(mm(with_bits(0xFF), x, n, k), plus, rtol=1e-13, atol=0)
    ok &= np.allclose(mm(with_bits(0x00), x, n, k), -plus, rtol=1e-13, atol=0)
    # complementing every bit negates the output; the residual is added once
    comp = a.copy()
    comp[:, :, :16] ^= 0xFF
    base = mm(aos, x, n, k)
    ok &= np.allclose(mm(comp.reshape(-1), x, n, k), -base, rtol=1e-13, atol=1e-13)
    r = np.random.default_rng(3).standard_normal((3, n))
    ok &= np.allclose(mm(aos, x, n, k, r) - base, r, rtol=0, atol=1e-12)
    zero = a.copy()
    zero[:, :, 16:] = 0
    ok &= np.array_equal(mm(zero.reshape(-1), x, n, k), np.zeros((3, n)))
    return bool(ok)


def pin_q1_scalar_loop(mm):
    ok = True
    for seed, (m, n, k) in enumerate([(1, 1, 128), (2, 3, 256), (3, 2, 384)]):
        c = G.random_case_q1(200 + seed, m, n, k, residual=True)
        ref = np.array(Q.matmul_scalar_q1(bytes(c["aos"]), c["x"].tolist(), n, k,
                                          c["residual"].tolist()))
        ok &= np.allclose(mm(c["aos"], c["x"], n, k, c["residual"]), ref, rtol=1e-12,
                          atol=1e-12)
    return bool(ok)


def _q1_mm(aos, x, n, k, residual=None):
    return O.matmul(aos, x, n, k, residual, fmt="q1")


def test_q1_block_size():
    assert Q.Q1_BLOCK_BYTES == 18 and Q.q1_aos_bytes(1, 128) == 18
    assert Q.q1_aos_bytes(4096, 4096) == 131072 * 18          # 2,359,296 B


def test_q1_hand_worked_blocks():
    assert pin_q1_hand_worked(Q.dequantize_q1)

    def deq_scalar(aos, n, k):
        return np.array(Q.dequantize_scalar_q1(bytes(aos), n, k))
    assert pin_q1_hand_worked(deq_scalar)
    assert pin_q1_unit_vectors(deq_scalar)


def test_q1_unit_vectors():
    assert pin_q1_unit_vectors(Q.dequantize_q1)


def test_q1_two_block_row_and_closed_forms():
    assert pin_q1_two_block_row(_q1_mm)
    assert pin_q1_closed_forms(_q1_mm)


def test_q1_matches_scalar_triple_loop():
    assert pin_q1_scalar_loop(_q1_mm)


def test_q1_entries_rows_and_swiglu_use_the_q1_decoder():
    n, k = 9, 256
    c = G.random_case_q1(210, 5, n, k, residual=True)
    full = O.matmul(c["aos"], c["x"], n, k, c["residual"], fmt="q1")
    rows, cols = np.array([0, 4, 2]), np.array([8, 0, 3])
    ref, _ = O.matmul_entries(c["aos"], c["x"], n, k, rows, cols, c["residual"], fmt="q1")
    assert np.allclose(ref, full[rows, cols], rtol=1e-13, atol=1e-13)
    ref2, _ = O.matmul_rows(c["aos"], c["x"], n, k, [1, 7], c["residual"], fmt="q1")
    assert np.allclose(ref2, full[:, [1, 7]], rtol=1e-13, atol=1e-13)
    s = G.swiglu_case_q1(211, 3, n, k)
    g = O.matmul(s["gate"], s["x"], n, k, fmt="q1")
    u = O.matmul(s["up"], s["x"], n, k, fmt="q1")
    assert np.allclose(O.gate_up_swiglu(s["gate"], s["up"], s["x"], n, k, fmt="q1"),
                       g * expit(g) * u, rtol=1e-12, atol=1e-15)
    with pytest.raises(ValueError):
        O.matmul(c["aos"], c["x"], n, k, fmt="q2")


def _mutant_q1(kind):
    def deq(aos, n, k, rows=None):
        blk = Q._blocks_q1(aos, n, k)
        qs = blk[:, :, :16]
        lo, hi = blk[:, :, 16].astype(np.uint16), blk[:, :, 17].astype(np.uint16)
        bits = lo | (hi << 8)
        if kind == "scale_big_endian":
            bits = hi | (lo << 8)
        d = O.f16_bits_to_float_array(bits)
        w = np.empty(qs.shape[:2] + (128,))
        for j in range(128):
            if kind == "msb_first":
                b = (qs[:, :, j >> 3] >> (7 - (j & 7))) & 1
            elif kind == "strided":
                b = (qs[:, :, j & 15] >> (j >> 4)) & 1
            else:
                b = (qs[:, :, j >> 3] >> (j & 7)) & 1
            val = np.where(b == 1, 1.0, -1.0)
            if kind == "sign_swapped":
                val = -val
            if kind == "zero_for_clear":
                val = np.where(b == 1, 1.0, 0.0)
            w[:, :, j] = val * (1.0 if kind == "scale_dropped" else d)
        return w.reshape(w.shape[0], -1)
    return deq


@pytest.mark.parametrize("kind", ["msb_first", "strided", "sign_swapped", "zero_for_clear",
                                  "scale_dropped", "scale_big_endian"])
def test_pins_catch_planted_q1_mistakes(kind):
    deq = _mutant_q1(kind)

    def mm(aos, x, n, k, residual=None):
        out = np.asarray(x, np.float64).reshape(-1, k) @ deq(aos, n, k).T
        return out if residual is None else np.asarray(residual, np.float64) + out
    results = [pin_q1_hand_worked(deq), pin_q1_unit_vectors(deq), pin_q1_two_block_row(mm),
               pin_q1_closed_forms(mm), pin_q1_scalar_loop(mm)]
    assert not all(results), kind
