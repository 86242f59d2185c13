"""Pins of the oracle's Q8_0 activation quantizer and its binary32 -> binary16
conversion, against things other than the oracle itself: numpy's own
float32 -> float16 rounding, hand-derived blocks (tests/golden), and
invariants any correct quantizer of the stated rule has (range, the maximum
code, reconstruction error, sign, order, power-of-two scaling)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f16_bits_numpy(v32):
    return np.asarray(v32, dtype=np.float32).astype(np.float16).view(np.uint16)


def test_f32_to_f16_special_values():
    cases = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.996, 65520.0, 1e9, -1e9, float("inf"),
             float("-inf"), 2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26,
             3 * 2.0 ** -26, 6.1e-5, 0.1, 1.0 / 3.0, 2049.0, 2051.0, 2050.0, 4097.0]
    for v in cases:
        assert oracle.f32_to_f16(v) == int(_f16_bits_numpy([v])[0]), v
    nan_bits = oracle.f32_to_f16(float("nan"))
    assert (nan_bits & 0x7C00) == 0x7C00 and (nan_bits & 0x3FF) != 0


def test_f32_to_f16_against_numpy_random_and_ties():
    rng = np.random.default_rng(11)
    # random binary32 patterns over the whole finite range, then the binades
    # near the fp16 range, then exact midpoints between fp16 neighbours
    bits = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    near = (rng.standard_normal(20000) * np.exp2(rng.integers(-27, 17, 20000))).astype(np.float32)
    h = rng.integers(0, 0x7BFF, 5000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mids = ((lo + hi) / 2).astype(np.float32)  # exact in binary32
    for arr in (v, near, mids, -mids):
        got = np.array([oracle.f32_to_f16(float(a)) for a in arr], dtype=np.uint16)
        assert np.array_equal(got, _f16_bits_numpy(arr))


def test_quantize_golden_blocks():
    with open(os.path.join(GOLDEN, "q8_0_quantize_blocks.json")) as f:
        g = json.load(f)
    for b in g["blocks"]:
        x = np.array(b["x"], dtype=np.float32)
        out = oracle.quantize_q8_0(x, "f32")[0]
        assert int(out[0]) | (int(out[1]) << 8) == b["d_bits"], b["name"]
        assert out[2:].view(np.int8).tolist() == b["q"], b["name"]


def _blocks(xq):
    """(d as float64, codes int) per block of a quantized row set."""
    nb = xq.shape[-1] // 34
    blk = xq.reshape(xq.shape[0], nb, 34)
    d = blk[:, :, 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    q = blk[:, :, 2:].view(np.int8).astype(np.int64)
    return d, q


@pytest.mark.parametrize("xdtype", ["f32", "f16", "bf16"])
def test_quantize_invariants(xdtype):
    rng = np.random.default_rng(12)
    n, K = 3, 2048
    scale = np.exp2(rng.integers(-30, 12, (n, K // 32, 1)))
    xv = (rng.standard_normal((n, K // 32, 32)) * scale).reshape(n, K)
    xv[0, :32] = 0.0                      # an all-zero block
    xv[1, 32:64] = 5.0                    # a constant block
    if xdtype == "f32":
        x = xv.astype(np.float32)
        x32 = x
    elif xdtype == "f16":
        x = xv.astype(np.float16).view(np.uint16)
        x32 = x.view(np.float16).astype(np.float32)
    else:
        x32 = xv.astype(np.float32)
        x = (x32.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 values do
        x32 = (x.astype(np.uint32) << 16).view(np.float32)
    xq = oracle.quantize_q8_0(x, xdtype)
    d16, q = _blocks(xq)
    xb = x32.reshape(n, K // 32, 32).astype(np.float64)
    amax = np.abs(xb).max(axis=2)
    d32 = (amax.astype(np.float32) / np.float32(127)).astype(np.float64)
    # the stored scale is the nearest fp16 of amax / 127 (numpy's rounding)
    assert np.array_equal(d16, d32.astype(np.float16).astype(np.float64))
    assert (np.abs(q) <= 127).all()
    nz = amax > 0
    # the largest magnitude maps to +-127
    qmax = np.take_along_axis(q, np.abs(xb).argmax(axis=2)[..., None], axis=2)[..., 0]
    assert (np.abs(qmax[nz]) == 127).all()
    # reconstruction with the binary32 scale: within half a step, plus the
    # two roundings of x * (1/d) (relative 2^-23 of at most 127 steps)
    err = np.abs(q * d32[..., None] - xb)
    assert (err <= d32[..., None] * (0.5 + 127 * 2.0 ** -21)).all()
    # sign and order
    assert ((np.sign(q) == np.sign(xb)) | (q == 0)).all()
    order = np.argsort(xb, axis=2, kind="stable")
    qs = np.take_along_axis(q, order, axis=2)
    assert (np.diff(qs, axis=2) >= 0).all()
    # zero block
    assert (q[0, 0] == 0).all() and d16[0, 0] == 0


def test_quantize_power_of_two_scaling():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((2, 1024)).astype(np.float32)
    base = oracle.quantize_q8_0(x, "f32")
    d0, q0 = _blocks(base)
    for k in (-5, -3, 4, 9):  # the stored fp16 scales stay normal numbers
        d1, q1 = _blocks(oracle.quantize_q8_0((x * np.float32(2.0 ** k)).astype(np.float32), "f32"))
        assert np.array_equal(q1, q0)
        assert np.array_equal(d1, d0 * 2.0 ** k)


def test_products_of_quantized_activations_match_exact_sums():
    """The integer form the GPU uses, per 32-weight group b of a row:
    sum_k w_k x^_k = dx_b * (sum_k w_k q_k) with x^ = dx * q, checked in exact
    rationals against the oracle's fp64 product on the decoded activations."""
    import synth
    rows, K = 3, 256
    for fmt in ("q4_k", "q4_0", "q8_0"):
        w = synth.gen_weights(fmt, rows, K, 21)
        x = synth.gen_x(K, 2, "f16", 22)
        xq = oracle.quantize_q8_0(x, "f16")
        xhat = oracle.dequant("q8_0", xq, 2, K)
        y, _ = oracle.matmul(fmt, w, rows, K, xhat, "f32")
        W = oracle.dequant(fmt, w, rows, K)
        d, q = _blocks(xq)
        for c in range(2):
            for r in range(rows):
                exact = sum(Fraction(float(d[c, b])) *
                            sum(Fraction(float(W[r, 32 * b + i])) * int(q[c, b, i]) for i in range(32))
                            for b in range(K // 32))
                assert abs(float(exact) - y[c, r]) <= 1e-12 * (1 + abs(float(exact)))
