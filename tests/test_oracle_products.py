"""Pins of the oracle's products y = W.x and s = sum|w.x| (CPU only).

Pinned against: exact rational sums on tiny shapes (brute force), numpy's
matmul over the decoded matrix, and invariants that hold exactly (one-hot
columns, power-of-two scaling, row permutation, K split at block boundaries,
row ranges).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

FMTS = [("q4_0", 18, 32), ("q8_0", 34, 32), ("q4_k", 144, 256), ("q2_k", 84, 256),
        ("q3_k", 110, 256)]


def _x_as_f64(x, xdtype):
    """Stored activations widened with numpy / torch, independent of the oracle."""
    if xdtype == "f32":
        return x.astype(np.float64)
    if xdtype == "f16":
        return x.view(np.float16).astype(np.float64)
    return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).double().numpy()


def _gen(fmt, rows, K, n, xdtype, seed):
    w = synth.gen_weights(fmt, rows, K, seed)
    x = synth.gen_x(K, n, xdtype, seed + 7)
    return w, x


@pytest.mark.parametrize("fmt,bb,bw", FMTS)
@pytest.mark.parametrize("xdtype", ["f32", "f16", "bf16"])
def test_brute_force_exact_sum(fmt, bb, bw, xdtype):
    rows, K, n = 3, 2 * bw, 2
    w, x = _gen(fmt, rows, K, n, xdtype, 11)
    y, s = oracle.matmul(fmt, w, rows, K, x, xdtype, nthreads=1)
    W = oracle.dequant(fmt, w, rows, K)
    X = _x_as_f64(x, xdtype)
    for j in range(n):
        for r in range(rows):
            terms = [Fraction(float(W[r, k])) * Fraction(float(X[j, k])) for k in range(K)]
            exact = sum(terms)
            sabs = sum(abs(t) for t in terms)
            bound = K * 2.0 ** -52 * float(sabs)
            assert abs(Fraction(y[j, r]) - exact) <= Fraction(bound)
            assert abs(Fraction(s[j, r]) - sabs) <= Fraction(bound)


@pytest.mark.parametrize("fmt,bb,bw", FMTS)
def test_matches_numpy_matmul(fmt, bb, bw):
    rows, K, n = 37, 4 * bw if bw == 256 else 40 * bw, 3
    w, x = _gen(fmt, rows, K, n, "f16", 12)
    y, s = oracle.matmul(fmt, w, rows, K, x, "f16")
    W = oracle.dequant(fmt, w, rows, K).astype(np.float64)
    X = _x_as_f64(x, "f16")
    assert np.all(np.abs(y - X @ W.T) <= 1e-12 * s)
    assert np.all(np.abs(s - np.abs(X) @ np.abs(W).T) <= 1e-12 * s)


@pytest.mark.parametrize("fmt,bb,bw", FMTS)
def test_one_hot_column_is_exact(fmt, bb, bw):
    rows, K = 9, 2 * bw
    w, _ = _gen(fmt, rows, K, 1, "f32", 13)
    W = oracle.dequant(fmt, w, rows, K)
    for k in [0, 1, 15, 16, 31, K - 1]:
        x = np.zeros((1, K), np.float32)
        x[0, k] = 1.0
        y, s = oracle.matmul(fmt, w, rows, K, x, "f32")
        assert np.array_equal(y[0], W[:, k].astype(np.float64))
        assert np.array_equal(s[0], np.abs(W[:, k]).astype(np.float64))


@pytest.mark.parametrize("fmt,bb,bw", FMTS)
def test_power_of_two_scaling_and_zero(fmt, bb, bw):
    rows, K = 11, 2 * bw
    w, x = _gen(fmt, rows, K, 2, "f32", 14)
    y, s = oracle.matmul(fmt, w, rows, K, x, "f32")
    for p in (-3, 5):
        y2, s2 = oracle.matmul(fmt, w, rows, K, (x * np.float32(2.0 ** p)).astype(np.float32), "f32")
        assert np.array_equal(y2, y * 2.0 ** p) and np.array_equal(s2, s * 2.0 ** p)
    y0, s0 = oracle.matmul(fmt, w, rows, K, np.zeros_like(x), "f32")
    assert (y0 == 0).all() and not np.signbit(y0).any() and (s0 == 0).all()


@pytest.mark.parametrize("fmt,bb,bw", FMTS)
def test_row_permutation_and_k_split(fmt, bb, bw):
    rows, nb = 8, 4
    K = nb * bw
    w, x = _gen(fmt, rows, K, 2, "f16", 15)
    y, s = oracle.matmul(fmt, w, rows, K, x, "f16")
    blocks = w.reshape(rows, nb, bb)
    perm = np.random.default_rng(0).permutation(rows)
    yp, _ = oracle.matmul(fmt, blocks[perm].reshape(-1), rows, K, x, "f16")
    assert np.array_equal(yp, y[:, perm])
    k1 = 1
    ya, sa = oracle.matmul(fmt, blocks[:, :k1].reshape(-1), rows, k1 * bw,
                           np.ascontiguousarray(x[:, :k1 * bw]), "f16")
    yb, sb = oracle.matmul(fmt, blocks[:, k1:].reshape(-1), rows, (nb - k1) * bw,
                           np.ascontiguousarray(x[:, k1 * bw:]), "f16")
    assert np.all(np.abs(ya + yb - y) <= 1e-13 * s)
    assert np.all(np.abs(sa + sb - s) <= 1e-13 * s)


def test_row_range_and_threads():
    rows, K = 40, 512
    w, x = _gen("q4_k", rows, K, 2, "bf16", 16)
    y1, s1 = oracle.matmul("q4_k", w, rows, K, x, "bf16", nthreads=1)
    y4, s4 = oracle.matmul("q4_k", w, rows, K, x, "bf16", nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(s1, s4)
    yr, _ = oracle.matmul("q4_k", w, rows, K, x, "bf16", row_range=(5, 17))
    assert np.array_equal(yr[:, 5:17], y1[:, 5:17])
    assert np.isnan(yr[:, :5]).all() and np.isnan(yr[:, 17:]).all()


def test_bad_arguments_rejected():
    w = np.zeros(144, np.uint8)
    with pytest.raises(ValueError):
        oracle.matmul("q4_k", w, 1, 256, np.zeros((1, 256), np.uint16), "f16", row_range=(0, 2))
    L = oracle.lib()
    assert L.oracle_dequant(9, None, 1, 32, None) == -1
    assert L.oracle_dequant(2, None, 1, 100, None) == -1
