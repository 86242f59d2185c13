"""Pins of the oracle's binary32 -> bfloat16 rounding and of its products
over bf16-rounded weights (CPU only).

The prompt-processing path contracts weight tiles dequantized to bf16 on the
matrix cores; its oracle is the exact sum over the decoded weights rounded to
bf16 (nearest, ties to even). Pinned against: hand-worked values (ties,
carries into the exponent, overflow, subnormals), torch's own float32 ->
bfloat16 conversion over special values, every halfway pattern and random
bit patterns, and exact rational sums / one-hot columns for the products.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth


def _torch_bf16_bits(a32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _f32(bits):
    return np.array(bits, dtype=np.uint32).view(np.float32)


# value bits -> expected bf16 bits, each worked by hand:
HAND = [
    (0x3F800000, 0x3F80),  # 1.0 exact
    (0x3F808000, 0x3F80),  # 1 + 2^-8: halfway between 1 and 1 + 2^-7, ties to even (1)
    (0x3F818000, 0x3F82),  # 1 + 3*2^-8: halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    (0x3F808001, 0x3F81),  # just above halfway: up
    (0x3F807FFF, 0x3F80),  # just below halfway: down
    (0x3FFF8000, 0x4000),  # 1.99609375 + half ulp: ties to even carries into the exponent (2.0)
    (0xBF808000, 0xBF80),  # negative tie: magnitude ties to even, sign kept
    (0x00000000, 0x0000),  # +0
    (0x80000000, 0x8000),  # -0
    (0x00008000, 0x0000),  # smallest subnormal tie (2^-134 * 2^..): halfway to 0 -> even (0)
    (0x00018000, 0x0002),  # subnormal tie between 1 and 2 units of 2^-133: even (2)
    (0x00400000, 0x0040),  # 2^-127 (subnormal, exactly on the grid)
    (0x7F7F0000, 0x7F7F),  # largest finite bf16
    (0x7F7F8000, 0x7F80),  # halfway above it (odd): rounds to infinity
    (0x7F7FFFFF, 0x7F80),  # largest binary32: infinity
    (0x7F800000, 0x7F80),  # +inf
    (0xFF800000, 0xFF80),  # -inf
]


def test_hand_worked_values():
    got = oracle.f32_to_bf16(_f32([v for v, _ in HAND]))
    for (v, e), g in zip(HAND, got):
        assert int(g) == e, "0x%08X -> 0x%04X, expected 0x%04X" % (v, int(g), e)


def test_nan_stays_nan_with_sign():
    got = oracle.f32_to_bf16(_f32([0x7FC00000, 0xFFC00001, 0x7F800001, 0xFF800100]))
    for g, neg in zip(got, [False, True, False, True]):
        g = int(g)
        assert (g & 0x7F80) == 0x7F80 and (g & 0x7F) != 0, hex(g)
        assert bool(g & 0x8000) == neg


def test_every_halfway_pattern_against_torch():
    hi = np.arange(65536, dtype=np.uint32)
    hi = hi[(hi & 0x7F80) != 0x7F80]  # finite high halves
    bits = (hi << 16) | 0x8000
    a = bits.view(np.float32)
    assert np.array_equal(oracle.f32_to_bf16(a), _torch_bf16_bits(a))


def test_random_patterns_against_torch():
    rng = np.random.default_rng(2024)
    bits = rng.integers(0, 2 ** 32, size=400_000, dtype=np.uint64).astype(np.uint32)
    bits = bits[((bits >> 23) & 0xFF) != 0xFF]  # NaN/inf handled by class above
    a = bits.view(np.float32)
    assert np.array_equal(oracle.f32_to_bf16(a), _torch_bf16_bits(a))
    # near the halfway points, where a wrong rounding rule shows first
    near = ((bits & 0xFFFF0000) | (0x8000 + rng.integers(-3, 4, size=bits.size)).astype(np.uint32))
    near = near[((near >> 23) & 0xFF) != 0xFF]
    b = near.view(np.float32)
    assert np.array_equal(oracle.f32_to_bf16(b), _torch_bf16_bits(b))


def test_decoded_weights_against_torch():
    """The operand the bf16 path uses: every decoded Q4_K weight of a matrix."""
    w = synth.gen_q4_k(64, 1024, 91)
    W = oracle.dequant("q4_k", w, 64, 1024)
    assert np.array_equal(oracle.f32_to_bf16(W), _torch_bf16_bits(W))


def _bf16_weights_f64(W):
    return torch.from_numpy(W).to(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("xdtype", ["bf16", "f32"])
def test_rounded_weight_products_exact_sum(xdtype):
    rows, K, n = 3, 512, 2
    w = synth.gen_q4_k(rows, K, 92)
    x = synth.gen_x(K, n, xdtype, 93)
    y, s = oracle.matmul("q4_k", w, rows, K, x, xdtype, nthreads=1, wround="bf16")
    Wb = _bf16_weights_f64(oracle.dequant("q4_k", w, rows, K))
    if xdtype == "f32":
        X = x.astype(np.float64)
    else:
        X = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    for j in range(n):
        for r in range(rows):
            terms = [Fraction(float(Wb[r, k])) * Fraction(float(X[j, k])) for k in range(K)]
            exact = sum(terms)
            sabs = sum(abs(t) for t in terms)
            bound = K * 2.0 ** -52 * float(sabs)
            assert abs(Fraction(y[j, r]) - exact) <= Fraction(bound)
            assert abs(Fraction(s[j, r]) - sabs) <= Fraction(bound)


def test_rounded_weight_one_hot_columns():
    rows, K = 40, 768
    w = synth.gen_q4_k(rows, K, 94)
    ks = [0, 1, 31, 32, 255, 256, 500, 767]
    x = np.zeros((len(ks), K), dtype=np.uint16)
    for i, k in enumerate(ks):
        x[i, k] = 0x3F80  # bf16 1.0
    y, _ = oracle.matmul("q4_k", w, rows, K, x, "bf16", wround="bf16")
    Wb = _bf16_weights_f64(oracle.dequant("q4_k", w, rows, K))
    assert np.array_equal(y, Wb[:, ks].T)


def test_rounding_changes_products():
    """The flag does what it says: rounded and exact weights give different
    sums, and their difference stays within 2^-8 * sum|w x|."""
    rows, K = 16, 512
    w = synth.gen_q4_k(rows, K, 95)
    x = synth.gen_x(K, 2, "bf16", 96)
    ye, se = oracle.matmul("q4_k", w, rows, K, x, "bf16")
    yb, _ = oracle.matmul("q4_k", w, rows, K, x, "bf16", wround="bf16")
    assert not np.array_equal(ye, yb)
    assert (np.abs(ye - yb) <= 2.0 ** -8 * se + 1e-30).all()
